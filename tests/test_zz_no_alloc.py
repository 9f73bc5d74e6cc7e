"""GPU check of the allocation-free entry point, kda_conv_verify_decode_noalloc, through the
raw C ABI: it keeps its counters in the library's static per-GPU scratch instead of a
caller's workspace, and must return exactly what kda_conv_verify_decode returns with a
workspace (the same kernels and launch) on two calls in a row, the second on a smaller
input, so that the second call runs on whatever the first left in the scratch.

For callers that cannot allocate device memory (graph capture, serving loops).
"""
import ctypes

import pytest
import torch

import linear_attention_decode_kda_amd as kda
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches_all, bit_view, say, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("o", "inter_ssm", "conv_window", "conv_state")


def _raw_noalloc(p, g, out):
    lib = kda.load()
    ptrs = [t.data_ptr() for t in (g["mixed_qkv"], g["conv_weight"], g["conv_state"], g["gate"], g["A_log"],
                                   g["dt_bias"], g["beta"], g["state"], out["o"], out["inter_ssm"],
                                   out["conv_window"])]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.kda_conv_verify_decode_noalloc(ctypes.byref(p), *[ctypes.c_void_p(x) for x in ptrs], stream)


def _both(w):
    """The same inputs through the workspace entry point and the allocation-free one."""
    inp = synth.make_inputs(w)
    p = kda.params_for(w)
    say(f"[gpu] noalloc {w.name} N={w.N} T={w.T} H={w.H} HV={w.HV} launch={kda.select_launch(p)}")
    base = to_dev(inp)
    g1 = {k: v.clone() for k, v in base.items()}
    o1 = kda.alloc_outputs(w)
    for t in o1.values():
        t.fill_(float("nan"))
    kda.run(p, g1, o1, kda.alloc_workspace(p))
    g2 = {k: v.clone() for k, v in base.items()}
    o2 = kda.alloc_outputs(w)
    for t in o2.values():
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    st = _raw_noalloc(p, g2, o2)
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    torch.cuda.synchronize()
    assert st == 0, kda.STATUS.get(st, st)
    assert after == before, "the allocation-free call allocated through torch"
    o1["conv_state"], o2["conv_state"] = g1["conv_state"], g2["conv_state"]
    for k in OUTS:
        assert torch.equal(bit_view(o2[k]), bit_view(o1[k])), f"{w.name}: {k} differs from the workspace call"
    err = assert_matches_all(w, inp, o2, what=f"noalloc {w.name}")
    say(f"[gpu] noalloc {w.name}: bit-identical to the workspace call, max-abs o={err['o']:.2e} "
        f"inter_ssm={err['inter_ssm']:.2e}")


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    # first: the queue schedule over 2048 units with two value heads per q/k head (ticket,
    # leave and arrival counters all used); second: a smaller grid call on the scratch the
    # first one left behind
    _both(synth.WORKLOADS["gva"])
    _both(synth.WORKLOADS["gva"].with_(N=5, seed=1102))


def test_noalloc_repeated_calls_and_the_size_limit():
    """Three more calls of different shapes back to back on one stream, then a shape that
    needs more counters than the scratch holds, which is refused before any launch."""
    for w in (synth.WORKLOADS["small_batch"], synth.WORKLOADS["tiny"],
              synth.WORKLOADS["large_batch"].with_(N=64, seed=1203)):
        _both(w)
    w = synth.Workload("too_big", N=4096, T=1, H=16, HV=16, K=128, V=128, dtype="bf16", gate="softplus", seed=1)
    p = kda.params_for(w)
    assert kda.workspace_bytes(p) > kda.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    lib = kda.load()
    st = lib.kda_conv_verify_decode_noalloc(ctypes.byref(p), *[ctypes.c_void_p(dummy.data_ptr())] * 11, None)
    assert st == -8
