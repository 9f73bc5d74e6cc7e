"""GPU robustness: determinism over many repeats, guard bands and NaN poisoning (a
memcheck/initcheck stand-in), error paths that must leave every buffer untouched,
workspace recovery, non-default streams, concurrent calls and graph replay.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request):
determinism stress (commit 2), multistream and graph replay, repeated chains
(Tests & Accuracy), stale last-arrival counters (code review).
"""
import ctypes

import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _setup(w, variant=kda.VARIANT_AUTO, **pkw):
    inp = synth.make_inputs(w)
    g = to_dev(inp)
    p = kda.params_for(w, variant=variant, **pkw)
    ws = kda.alloc_workspace(p)
    out = kda.alloc_outputs(w)
    return inp, g, p, ws, out


@pytest.mark.parametrize("name,reps", [("small_batch", 10000), ("gva", 2000), ("large_batch", 10000)])
def test_determinism_repeats(name, reps):
    """Repeated calls on the same inputs give bitwise identical outputs. conv_state is
    rolled in place, so it is restored from a pristine copy before each call. On
    large_batch AUTO runs the queue schedule, whose unit-to-CU assignment changes from
    call to call while the bits must not (and whose counters must reset every call)."""
    w = synth.WORKLOADS[name]
    say(f"[gpu] determinism {name} x{reps}")
    inp, g, p, ws, out = _setup(w)
    cs0 = g["conv_state"].clone()
    kda.run(p, g, out, ws)
    ref = {k: v.clone() for k, v in out.items()}
    ref_cs = g["conv_state"].clone()
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for i in range(reps):
        g["conv_state"].copy_(cs0)
        kda.run(p, g, out, ws)
        if i % 97 == 0 or i == reps - 1:  # full compare on a sample of repeats, cheap checksum on all
            for k in ref:
                bad += (out[k].view(torch.int16 if out[k].element_size() == 2 else torch.int32)
                        != ref[k].view(torch.int16 if ref[k].element_size() == 2 else torch.int32)).sum()
            bad += (g["conv_state"].view(torch.int16) != ref_cs.view(torch.int16)).sum()
        else:
            bad += (out["o"].view(torch.int16) != ref["o"].view(torch.int16)).sum()
            bad += (out["inter_ssm"][:, -1] != ref["inter_ssm"][:, -1]).sum()
    torch.cuda.synchronize()
    assert int(bad) == 0
    assert_matches(w.with_(N=2), {k: v[:2] for k, v in {**out, "conv_state": g["conv_state"]}.items()},
                   oracle.verify_workload(w.with_(N=2), {k: (v[:2] if v.dim() > 1 and v.shape[0] == w.N else v)
                                                          for k, v in inp.items()}), what="determinism")


def _guarded(shape, dtype, fill, guard_elems=4096):
    """A tensor view with guard bands on both sides of a known pattern."""
    n = 1
    for s in shape:
        n *= s
    buf = torch.empty(n + 2 * guard_elems, dtype=dtype, device="cuda")
    pattern = torch.arange(guard_elems, device="cuda").to(dtype)
    buf[:guard_elems] = pattern
    buf[-guard_elems:] = pattern
    view = buf[guard_elems:guard_elems + n].view(shape)
    view.fill_(fill)
    return buf, view, pattern


@pytest.mark.parametrize("w,variant", [(synth.WORKLOADS["gva"].with_(N=5), kda.VARIANT_SMALL),
                                       (synth.WORKLOADS["gva"].with_(N=5), kda.VARIANT_LARGE),
                                       (synth.WORKLOADS["tiny"], kda.VARIANT_AUTO)])
def test_guard_bands_and_nan_poison(w, variant):
    """Every output element is written (no NaN survives) and nothing outside the
    buffers changes (guard bands keep their pattern)."""
    say(f"[gpu] guards {w.name} N={w.N} variant={variant}")
    inp = synth.make_inputs(w)
    p = kda.params_for(w, variant=variant)
    dt = w.torch_dtype
    bufs = {}
    views = {}
    for k, v in inp.items():
        bufs[k], views[k], _ = _guarded(tuple(v.shape), v.dtype, 0.0)
        views[k].copy_(v.cuda())
    for k, shape, dtype in (("o", (w.N, w.T, w.HV, w.V), dt), ("inter_ssm", (w.N, w.T, w.HV, w.K, w.V), torch.float32),
                            ("conv_window", (w.N, w.T, w.C, 3), dt)):
        bufs[k], views[k], _ = _guarded(shape, dtype, float("nan"))
    wsb = kda.workspace_bytes(p)
    bufs["ws"], views["ws"], _ = _guarded((wsb,), torch.uint8, 0)
    before = {k: b.clone() for k, b in bufs.items()}
    kda.kda_conv_verify_decode(p, views["mixed_qkv"], views["conv_weight"], views["conv_state"], views["gate"],
                               views["A_log"], views["dt_bias"], views["beta"], views["state"], views["o"],
                               views["inter_ssm"], views["conv_window"], views["ws"])
    torch.cuda.synchronize()
    G = 4096
    for k, b in bufs.items():
        n = b.numel() - 2 * G
        assert torch.equal(b[:G], before[k][:G]) and torch.equal(b[G + n:], before[k][G + n:]), f"guard of {k}"
    for k in ("mixed_qkv", "conv_weight", "gate", "A_log", "dt_bias", "beta", "state"):
        assert torch.equal(bufs[k], before[k]), f"read-only input {k} changed"
    assert torch.count_nonzero(views["ws"]) == 0, "counters not left at zero"
    got = {k: views[k] for k in ("o", "inter_ssm", "conv_window", "conv_state")}
    assert_matches(w, got, oracle.verify_workload(w, inp), what="guarded")


def test_error_paths_leave_buffers_untouched():
    """Rejected calls return their status, launch nothing and write nothing."""
    w = synth.WORKLOADS["gva"].with_(N=3)
    inp, g, p, ws, out = _setup(w)
    for v in out.values():
        v.fill_(1.5)
    snap = {k: v.clone() for k, v in {**g, **out}.items()}
    lib = kda.load()
    base = [t.data_ptr() for t in (g["mixed_qkv"], g["conv_weight"], g["conv_state"], g["gate"], g["A_log"],
                                    g["dt_bias"], g["beta"], g["state"], out["o"], out["inter_ssm"],
                                    out["conv_window"], ws)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def raw(pp, ptrs=base, wsb=ws.numel()):
        return lib.kda_conv_verify_decode(ctypes.byref(pp), *[ctypes.c_void_p(x) for x in ptrs], wsb, stream)

    bad = kda.params_for(w)
    bad.T = kda.MAX_T + 1
    assert raw(bad) == -2
    bad = kda.params_for(w)
    bad.HV = w.H * 3 + 1
    assert raw(bad) == -2
    bad = kda.params_for(w)
    bad.K = bad.V = 96
    assert raw(bad) == -3
    ptrs = list(base)
    ptrs[0] += 2  # misaligned mixed_qkv
    assert raw(p, ptrs) == -4
    ptrs = list(base)
    ptrs[8] = 0  # NULL o
    assert raw(p, ptrs) == -1
    assert raw(p, wsb=16) == -5  # workspace too small
    ptrs = list(base)
    ptrs[9] = ptrs[7]  # inter_ssm over state
    assert raw(p, ptrs) == -7
    torch.cuda.synchronize()
    for k, v in {**g, **out}.items():
        assert torch.equal(v, snap[k]), f"{k} changed by a rejected call"


def test_stale_counters_recovered_by_reset():
    """Counters left non-zero (an interrupted call) may misplace the q/k conv_state
    write; kda_workspace_reset restores correct behaviour."""
    w = synth.WORKLOADS["gva"].with_(N=4)
    inp, g, p, ws, out = _setup(w, kda.VARIANT_SMALL)
    cs0 = g["conv_state"].clone()
    ws.fill_(3)  # garbage counts: never faults, may only misplace the write
    kda.run(p, g, out, ws)
    g["conv_state"].copy_(cs0)
    kda.workspace_reset(ws)
    kda.run(p, g, out, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws) == 0
    assert_matches(w, {**out, "conv_state": g["conv_state"]}, oracle.verify_workload(w, inp), what="after reset")


@pytest.mark.parametrize("qa", [0, 2])
def test_non_default_stream_and_concurrent_calls(qa):
    """Overlapping calls on two streams with their own workspaces; with qa = 2 the first
    runs the queue schedule over 2048 units while the second runs beside it."""
    wa = synth.WORKLOADS["gva"].with_(N=64 if qa else 6)
    wb = synth.WORKLOADS["small_batch"].with_(N=5, seed=77)
    say(f"[gpu] two streams, schedule {qa}")
    ia, ga, pa, wsa, oa = _setup(wa, schedule=qa)
    ib, gb, pb, wsb, ob = _setup(wb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):  # alternating, overlapping launches on two streams
        with torch.cuda.stream(sa):
            kda.run(pa, ga, oa, wsa)
        with torch.cuda.stream(sb):
            kda.run(pb, gb, ob, wsb)
        torch.cuda.synchronize()
        ga["conv_state"].copy_(ia["conv_state"].cuda())
        gb["conv_state"].copy_(ib["conv_state"].cuda())
    with torch.cuda.stream(sa):
        kda.run(pa, ga, oa, wsa)
    with torch.cuda.stream(sb):
        kda.run(pb, gb, ob, wsb)
    torch.cuda.synchronize()
    assert_matches(wa, {**oa, "conv_state": ga["conv_state"]}, oracle.verify_workload(wa, ia), what="stream a")
    assert_matches(wb, {**ob, "conv_state": gb["conv_state"]}, oracle.verify_workload(wb, ib), what="stream b")


@pytest.mark.parametrize("N,sched", [(8, 0), (64, 2)])
def test_graph_replay_matches_eager(N, sched):
    """Capture one call in a HIP graph; every replay (conv_state restored eagerly in
    between) equals the eager result bit for bit. With the queue schedule (2048 units over
    the resident workgroups) each replay also relies on the previous one having zeroed the
    queue counters."""
    w = synth.WORKLOADS["gva"].with_(N=N)
    say(f"[gpu] graph replay gva N={N} schedule {sched}")
    inp, g, p, ws, out = _setup(w, schedule=sched)
    cs0 = g["conv_state"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.run(p, g, out, ws)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    eager_cs = g["conv_state"].clone()
    graph = torch.cuda.CUDAGraph()
    g["conv_state"].copy_(cs0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        kda.run(p, g, out, ws)
    for rep in range(5):
        g["conv_state"].copy_(cs0)
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], eager[k]), (rep, k)
        assert torch.equal(g["conv_state"], eager_cs), rep
    assert_matches(w, {**eager, "conv_state": eager_cs}, oracle.verify_workload(w, inp), what="graph")


def test_prepared_call_matches_plain_call():
    """PreparedVerify (checks once, cached pointers) returns the same bits as the plain
    call, call after call on a chain of rolled conv caches, and matches the oracle."""
    w = synth.WORKLOADS["gva"].with_(N=8)
    say("[gpu] prepared call vs plain call, gva N=8, 3 chained calls")
    inp, g, p, ws, out = _setup(w)
    g2 = {k: v.clone() for k, v in g.items()}
    out2 = kda.alloc_outputs(w)
    ws2 = kda.alloc_workspace(p)
    call = kda.PreparedVerify(p, g2, out2, ws2)
    for i in range(3):
        kda.run(p, g, out, ws)
        call()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k].view(torch.int16 if out[k].element_size() == 2 else torch.int32),
                               out2[k].view(torch.int16 if out2[k].element_size() == 2 else torch.int32)), (i, k)
        assert torch.equal(g["conv_state"].view(torch.int16), g2["conv_state"].view(torch.int16)), i
        if i == 0:
            assert_matches(w, {**out2, "conv_state": g2["conv_state"]}, oracle.verify_workload(w, inp),
                           what="prepared")
