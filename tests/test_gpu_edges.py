"""Edge shapes of the verify step on the GPU, through the C ABI.

* An empty batch (N = 0) is a no-op: the call succeeds and touches nothing.
* The widest q/k sharing: one q/k head for 64 value heads, so 64 to 256 workgroups read
  (and one of them rolls) the same q/k conv cache, on the grid in whole-V column groups,
  on the 32-column split and on the queue; three calls in a row on one workspace, which
  must be all zero again after each call (the arrival counters reset themselves).
* The longest draft the library takes (T = 16) on the queue schedule with shared q/k heads.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), PR
description (HV >= H, any T >= 1, last-arrival counters) and Tests & Accuracy (edge shapes).
"""
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches, say, to_dev

pytestmark = pytest.mark.gpu


def test_empty_batch_is_a_no_op():
    w = synth.WORKLOADS["small_batch"].with_(N=0)
    inp = to_dev(synth.make_inputs(w))
    keep = {k: v.clone() for k, v in inp.items()}
    out = kda.alloc_outputs(w)
    p = kda.params_for(w)
    ws = kda.alloc_workspace(p)
    say("[gpu] empty batch N=0")
    kda.run(p, inp, out, ws)
    torch.cuda.synchronize()
    for k, v in inp.items():
        assert torch.equal(v, keep[k]), k
    assert int(ws.count_nonzero()) == 0


def _three_calls(w, **launch):
    """Three calls on one workspace, each checked against the oracle; the workspace must
    be all zero after each."""
    p = kda.params_for(w, **launch)
    ws = kda.alloc_workspace(p)
    for call in range(3):
        inp = synth.make_inputs(w, seed=w.seed + call)
        ref = oracle.verify_workload(w, inp)
        g = to_dev(inp)
        out = kda.alloc_outputs(w)
        for t in out.values():
            t.fill_(float("nan"))
        say(f"[gpu] {w.name} call {call} launch={kda.select_launch(p)}")
        kda.run(p, g, out, ws)
        torch.cuda.synchronize()
        out["conv_state"] = g["conv_state"]
        assert_matches(w, out, ref, what=f"{w.name} call {call} {launch}")
        assert int(ws.count_nonzero()) == 0, f"{w.name} call {call}: workspace not left zero"


@pytest.mark.parametrize("launch", [dict(), dict(variant=kda.VARIANT_SMALL), dict(schedule=2)],
                         ids=["auto-grid", "small-32col", "queue"])
def test_one_qk_head_for_64_value_heads(launch):
    w = synth.Workload("g64", N=3, T=5, H=1, HV=64, K=128, V=128, dtype="bf16", gate="softplus", seed=640)
    _three_calls(w, **launch)


def test_longest_draft_on_the_queue():
    w = synth.Workload("t16q", N=20, T=16, H=4, HV=8, K=128, V=128, dtype="bf16", gate="safe", seed=160)
    p = kda.params_for(w, schedule=2)
    assert kda.select_launch(p)["schedule"] == 2
    _three_calls(w, schedule=2)
