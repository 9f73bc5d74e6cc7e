"""GPU checks of the queue schedule: resident workgroups pulling units from a counter in
the workspace. The schedule only changes which CU runs a unit and when, so its outputs
must equal the grid's bit for bit, on every call of a chain that reuses one workspace
(the last workgroup out zeroes the counters for the next call).

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), PR
description: one workgroup per (sequence, value head) unit, and last-arrival counters
deciding which workgroup writes the shared q/k conv cache; the counters here take the
same role for the queue.
"""
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches, assert_matches_all, say, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("o", "inter_ssm", "conv_window", "conv_state")


def W(N, T, H, HV, K=128, V=128, dtype="bf16", gate="softplus", seed=21):
    return synth.Workload(f"queue{N}x{T}x{H}x{HV}x{K}", N=N, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, gate=gate,
                          seed=seed)


def _chain(w, inp, calls, **pkw):
    """`calls` back-to-back calls on one workspace, each from the same inputs (conv_state is
    rolled in place, so each call gets a fresh copy); returns every call's outputs."""
    p = kda.params_for(w, **pkw)
    say(f"[gpu] {w.name} {w.dtype} {w.gate} {pkw} -> {kda.select_launch(p)} x{calls}")
    base = to_dev(inp)
    ws = kda.alloc_workspace(p)
    res = []
    for _ in range(calls):
        g = {k: v.clone() for k, v in base.items()}
        out = kda.alloc_outputs(w)
        for t in out.values():
            t.fill_(float("nan"))
        kda.run(p, g, out, ws)
        out["conv_state"] = g["conv_state"]
        res.append(out)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0, "the counters must be zero again after each call"
    return res


CASES = [
    # (workload, queue launch): many rounds per resident workgroup, shared and unshared q/k
    # heads, each column grouping and store policy, a cap the kernel cannot reach (more
    # workgroups than fit: the late ones find the queue drained), and no cap at all
    (W(96, 4, 32, 32), dict(tile_columns=128, max_wg_per_cu=1)),
    (W(96, 4, 32, 32, gate="safe"), dict(tile_columns=128, max_wg_per_cu=1, column_groups=2, store_policy=2)),
    (W(96, 4, 32, 32), dict(tile_columns=128, max_wg_per_cu=2, column_groups=4)),
    (W(48, 3, 16, 64), dict(tile_columns=128, max_wg_per_cu=1)),
    (W(48, 3, 16, 64), dict(tile_columns=128, max_wg_per_cu=1, column_groups=2)),
    (W(64, 1, 32, 32), dict(tile_columns=128, max_wg_per_cu=1, column_groups=4)),
    (W(40, 8, 16, 32, gate="safe"), dict(tile_columns=128, max_wg_per_cu=8, store_policy=2)),
    (W(24, 8, 16, 32, dtype="f32"), dict(tile_columns=128, max_wg_per_cu=1)),
    (W(64, 4, 8, 16, K=64, V=64), dict(max_wg_per_cu=1)),
    (W(300, 2, 4, 8, K=16, V=16, dtype="f32"), dict(max_wg_per_cu=1)),
]


@pytest.mark.parametrize("w,launch", CASES, ids=[f"{c[0].name}-{c[0].dtype}-{c[0].gate}-{i}" for i, c in
                                                 enumerate(CASES)])
def test_queue_equals_grid_on_every_call(w, launch):
    inp = synth.make_inputs(w)
    grid = _chain(w, inp, 1, schedule=1, **launch)[0]
    queue = _chain(w, inp, 3, schedule=2, **launch)
    for i, q in enumerate(queue):
        for k in OUTS:
            assert torch.equal(q[k], grid[k]), (i, k)
    assert_matches_all(w, inp, queue[-1], what=f"queue {w.name}")


def test_queue_with_fewer_units_than_resident_slots():
    """A grid of only the units (fewer than the CUs): every workgroup takes one unit by its
    index and finds the queue empty."""
    w = W(3, 4, 2, 4)
    inp = synth.make_inputs(w)
    out = _chain(w, inp, 2, schedule=2)
    for o in out:
        assert_matches(w, o, oracle.verify_workload(w, inp), what="queue, 12 units")


def test_queue_on_the_large_batch_workload_matches_the_grid():
    """The large-batch workload (N=256, T=4, H=HV=32) on the queue: identical to the grid on
    every call, and every sequence matches the oracle."""
    w = synth.WORKLOADS["large_batch"]
    inp = synth.make_inputs(w)
    queue = _chain(w, inp, 2, schedule=2)
    grid = _chain(w, inp, 1, schedule=1)[0]
    for q in queue:
        for k in OUTS:
            assert torch.equal(q[k], grid[k]), k
    del grid
    say("[gpu] large_batch queue: oracle on all 256 sequences")
    assert_matches_all(w, inp, queue[0], what="large_batch queue")
