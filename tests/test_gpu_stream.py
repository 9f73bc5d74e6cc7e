"""GPU checks of the stream schedule: the queue schedule with a producer wave per workgroup
that loads each unit's inputs and state tile into LDS (LDS-direct loads) while the compute
waves run the unit before it. Like the queue, it only changes which CU runs a unit and
when, so its outputs must equal the grid's bit for bit, on every call of a chain that
reuses one workspace, with either point at which the producer loads the next state tile.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), PR
description (large_batch: the state is prefetched; last-arrival counters deciding which
workgroup writes the shared q/k conv cache, which the producer takes over here).
"""
import pytest
import torch

import linear_attention_decode_kda_amd as kda
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches_all, say, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("o", "inter_ssm", "conv_window", "conv_state")


def W(N, T, H, HV, dtype="bf16", gate="softplus", seed=31):
    return synth.Workload(f"stream{N}x{T}x{H}x{HV}", N=N, T=T, H=H, HV=HV, K=128, V=128, dtype=dtype, gate=gate,
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
    # many units per resident workgroup, one value head per q/k head
    (W(96, 4, 32, 32), 1),
    (W(96, 4, 32, 32, gate="safe"), 2),
    # shared q/k heads: 4 and 64 value heads per q/k head (the producer counts each unit in)
    (W(48, 3, 16, 64, gate="safe"), 2),
    (W(20, 4, 1, 64), 2),
    # the largest staging record: T = 8 (bf16), and fp32 inputs at T = 8 (155 KiB of LDS)
    (W(40, 8, 16, 32, gate="safe"), 1),
    (W(40, 8, 16, 32), 2),
    (W(24, 8, 16, 32, dtype="f32"), 2),
    # one and two tokens: the producer has the least slack
    (W(64, 1, 32, 32), 1),
    (W(64, 1, 32, 32), 2),
    (W(64, 2, 16, 32, dtype="f32"), 1),
    # fewer units than resident workgroups: each takes one unit and finds the queue empty
    (W(7, 5, 4, 12, dtype="f32"), 2),
    (W(1, 3, 2, 2), 1),
]


@pytest.mark.parametrize("w,prefetch", CASES, ids=[f"{c[0].name}-{c[0].dtype}-{c[0].gate}-p{c[1]}" for c in CASES])
def test_stream_equals_grid_on_every_call(w, prefetch):
    inp = synth.make_inputs(w)
    grid = _chain(w, inp, 1, schedule=1, tile_columns=128)[0]
    stream = _chain(w, inp, 3, schedule=3, prefetch=prefetch)
    for i, q in enumerate(stream):
        for k in OUTS:
            assert torch.equal(q[k], grid[k]), (i, k)
    assert_matches_all(w, inp, stream[-1], what=f"stream {w.name}")


@pytest.mark.parametrize("name", ["gva", "large_batch"])
def test_auto_stream_on_the_named_workloads_matches_the_grid(name):
    """gva and large_batch, where AUTO picks the stream (state loaded at the start of the
    unit before): identical to the grid on every call, the other prefetch point gives the
    same bits, and every sequence matches the oracle."""
    w = synth.WORKLOADS[name]
    p = kda.params_for(w)
    assert kda.select_launch(p)["schedule"] == 3 and kda.select_launch(p)["prefetch"] == 2
    inp = synth.make_inputs(w)
    stream = _chain(w, inp, 2)
    other = _chain(w, inp, 1, prefetch=1)[0]
    grid = _chain(w, inp, 1, schedule=1)[0]
    for q in stream + [other]:
        for k in OUTS:
            assert torch.equal(q[k], grid[k]), k
    del grid, other
    say(f"[gpu] {name} stream: oracle on all {w.N} sequences")
    assert_matches_all(w, inp, stream[0], what=f"{name} stream")
