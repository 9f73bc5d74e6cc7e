"""GPU parity of the pooled verify step and the accept (commit) step.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request),
PR description: conv_state_indices, cache_indices and intermediate_state_indices,
normalised independently; per-token snapshots for rolling back to the accepted prefix.
Tests & Accuracy: independent, non-contiguous state indices; repeated verify chains.
"""
import random

import numpy as np
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import TOL, bits, say

pytestmark = pytest.mark.gpu


def W(N, T, H, HV, K=128, V=128, dtype="bf16", gate="softplus", seed=9):
    return synth.Workload(f"pool{N}x{T}x{H}x{HV}x{K}", N=N, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, gate=gate,
                          seed=seed)


def _gm(w):
    return oracle.GATE_SAFE if w.gate == "safe" else oracle.GATE_SOFTPLUS


def _pooled_case(w, slots, seed, pad=()):
    """Pools larger than N, rows picked at random without repeats; ``pad`` sequences get -1."""
    inp = synth.make_inputs(w)
    g = torch.Generator().manual_seed(seed)
    Pc, Ps, Pi = slots
    cs_idx = torch.randperm(Pc, generator=g)[: w.N].to(torch.int32)
    st_idx = torch.randperm(Ps, generator=g)[: w.N].to(torch.int32)
    in_idx = torch.randperm(Pi, generator=g)[: w.N].to(torch.int32)
    for n in pad:
        st_idx[n] = -1
    dt = w.torch_dtype
    cs_pool = torch.randn(Pc, w.C, 3, generator=g).to(dt)
    st_pool = torch.randn(Ps, w.HV, w.K, w.V, generator=g) * 0.1
    cs_pool[cs_idx.long()] = inp["conv_state"]
    keep = st_idx >= 0
    st_pool[st_idx[keep].long()] = inp["state"][keep]
    o0 = torch.randn(w.N, w.T, w.HV, w.V, generator=g).to(dt)
    is0 = torch.randn(Pi, w.T, w.HV, w.K, w.V, generator=g)
    cw0 = torch.randn(Pi, w.T, w.C, 3, generator=g).to(dt)
    pinp = dict(inp)
    pinp["conv_state"], pinp["state"] = cs_pool, st_pool
    idx = {"conv_state_indices": cs_idx, "cache_indices": st_idx, "intermediate_state_indices": in_idx}
    init = {"o": o0, "inter_ssm": is0, "conv_window": cw0}
    return pinp, idx, init


def _run_pooled(w, pinp, idx, init, variant=kda.VARIANT_AUTO, **pkw):
    say(f"[gpu] pooled {w.name} {w.dtype} {w.gate} variant={variant} {pkw}")
    p = kda.params_for(w, variant=variant, **pkw)
    d = {k: v.cuda() for k, v in pinp.items()}
    di = {k: v.cuda() for k, v in idx.items()}
    out = {k: v.cuda() for k, v in init.items()}
    pools = kda.make_pools(w.N, di["conv_state_indices"], di["cache_indices"], di["intermediate_state_indices"],
                           d["conv_state"].shape[0], d["state"].shape[0], out["inter_ssm"].shape[0])
    ws = kda.alloc_workspace(p)
    kda.kda_conv_verify_decode_pooled(p, pools, d["mixed_qkv"], d["conv_weight"], d["conv_state"], d["gate"],
                                      d["A_log"], d["dt_bias"], d["beta"], d["state"], out["o"],
                                      out["inter_ssm"], out["conv_window"], ws)
    torch.cuda.synchronize()
    out["conv_state"] = d["conv_state"]
    return out, d, di, pools, p


def _compare(w, got, ref):
    dt = w.torch_dtype
    assert np.array_equal(bits(got["conv_window"]), bits(torch.from_numpy(ref["conv_window"]).to(dt)))
    assert np.array_equal(bits(got["conv_state"]), bits(torch.from_numpy(ref["conv_state"]).to(dt)))
    eo = np.abs(got["o"].float().cpu().numpy() - ref["o"]).max()
    es = np.abs(got["inter_ssm"].cpu().numpy() - ref["inter_ssm"]).max()
    assert eo <= TOL and es <= TOL, (eo, es)


CASES = [
    (W(5, 4, 2, 4), (9, 7, 11), (), kda.VARIANT_SMALL),
    (W(5, 4, 2, 4, gate="safe"), (9, 7, 11), (1, 3), kda.VARIANT_LARGE),
    (W(3, 2, 1, 2, K=16, V=16, dtype="f32"), (4, 5, 6), (0,), kda.VARIANT_AUTO),
    (W(4, 8, 2, 2, K=64, V=64), (8, 4, 5), (2,), kda.VARIANT_AUTO),
]


@pytest.mark.parametrize("w,slots,pad,variant", CASES, ids=[f"{c[0].name}-pad{len(c[2])}-v{c[3]}" for c in CASES])
def test_pooled_verify_matches_oracle(w, slots, pad, variant):
    pinp, idx, init = _pooled_case(w, slots, seed=5, pad=pad)
    got, *_ = _run_pooled(w, pinp, idx, init, variant)
    ref = oracle.verify_pooled(pinp, {**idx, **init}, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    _compare(w, got, ref)


@pytest.mark.parametrize("launch", [dict(tile_columns=128, max_wg_per_cu=1),
                                    dict(tile_columns=32, max_wg_per_cu=4),
                                    dict(tile_columns=64, max_wg_per_cu=2),
                                    dict(tile_columns=128, max_wg_per_cu=1, column_groups=4),
                                    dict(tile_columns=128, max_wg_per_cu=1, schedule=2),
                                    dict(tile_columns=128, max_wg_per_cu=1, column_groups=2, schedule=2),
                                    dict(tile_columns=128, schedule=3, prefetch=1),
                                    dict(tile_columns=128, schedule=3, prefetch=2)])
def test_capped_grid_matches_oracle_and_uncapped(launch):
    """A workgroups-per-CU cap on a grid much larger than the part holds at once (padding
    sequences among them), or the queue or stream schedule pulling those units (padding
    units skip and hand on their ticket; the stream's producer skips them without a load),
    returns the bits of the uncapped grid and matches the oracle."""
    w = W(48, 3, 2, 8, gate="safe")  # 384 units of whole V: more than a persistent grid
    pinp, idx, init = _pooled_case(w, (60, 50, 70), seed=11, pad=(0, 17, 47))
    base, *_ = _run_pooled(w, pinp, idx, init, tile_columns=launch["tile_columns"])
    got, *_ = _run_pooled(w, pinp, idx, init, **launch)
    for k in ("o", "inter_ssm", "conv_window", "conv_state"):
        assert np.array_equal(bits(got[k]), bits(base[k])), k
    ref = oracle.verify_pooled(pinp, {**idx, **init}, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    _compare(w, got, ref)


def test_pooled_identity_equals_dense_call():
    w = W(6, 3, 2, 4)
    inp = synth.make_inputs(w)
    p = kda.params_for(w)
    a = {k: v.cuda() for k, v in inp.items()}
    b = {k: v.cuda() for k, v in inp.items()}
    oa, ob = kda.alloc_outputs(w), kda.alloc_outputs(w)
    kda.run(p, a, oa, kda.alloc_workspace(p))
    pools = kda.make_pools(w.N)
    kda.kda_conv_verify_decode_pooled(p, pools, b["mixed_qkv"], b["conv_weight"], b["conv_state"], b["gate"],
                                      b["A_log"], b["dt_bias"], b["beta"], b["state"], ob["o"], ob["inter_ssm"],
                                      ob["conv_window"], kda.alloc_workspace(p))
    torch.cuda.synchronize()
    for k in oa:
        assert torch.equal(oa[k], ob[k]), k
    assert torch.equal(a["conv_state"], b["conv_state"])


@pytest.mark.parametrize("w", [W(5, 4, 2, 4, gate="safe"), W(3, 3, 1, 1, K=16, V=16, dtype="f32")])
def test_commit_matches_oracle_and_prefix_verify(w):
    """Verify -> commit on the GPU against the oracle's own verify -> commit on the same
    inputs (the state within the 2e-3 bar, the conv cache bit-exact). On the GPU itself the
    commit is a bit copy: each committed state row holds its accepted snapshot, every other
    state row keeps its bits; and accepting a tokens gives the state and conv cache a fresh
    verify of just those a tokens produces."""
    slots = (w.N + 3, w.N + 2, w.N + 4)
    pinp, idx, init = _pooled_case(w, slots, seed=7)
    out, d, di, pools, p = _run_pooled(w, pinp, idx, init)
    acc = torch.tensor([(n % w.T) + 1 for n in range(w.N)], dtype=torch.int32)
    acc[0] = 0  # nothing accepted
    state_before = d["state"].clone()
    kda.verify_commit(p, pools, acc.cuda(), out["inter_ssm"], out["conv_window"], d["state"], d["conv_state"])
    torch.cuda.synchronize()
    rv = oracle.verify_pooled(pinp, {**idx, **init}, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    rc = oracle.commit(acc, idx, rv["inter_ssm"], rv["conv_window"], pinp["state"], rv["conv_state"], T=w.T)
    assert np.abs(d["state"].cpu().numpy() - rc["state"]).max() <= TOL
    assert np.array_equal(bits(d["conv_state"]), bits(torch.from_numpy(rc["conv_state"]).to(w.torch_dtype)))
    st_i, in_i = idx["cache_indices"], idx["intermediate_state_indices"]
    committed = set()
    for n in range(w.N):
        a, row = int(acc[n]), int(st_i[n])
        if a >= 1:
            committed.add(row)
            assert torch.equal(d["state"][row], out["inter_ssm"][int(in_i[n]), a - 1]), n
    for row in range(slots[1]):
        if row not in committed:
            assert torch.equal(d["state"][row], state_before[row]), row
    # accepted prefix: a dense verify of the first a tokens from the original inputs
    inp = synth.make_inputs(w)
    for n in range(1, w.N):
        a = int(acc[n])
        wa = w.with_(N=1, T=a)
        one = {k: (v[n:n + 1, :a].contiguous() if k in ("mixed_qkv", "gate", "beta") else
                   v[n:n + 1].contiguous() if k in ("conv_state", "state") else v).cuda()
               for k, v in inp.items()}
        po = kda.alloc_outputs(wa)
        pp = kda.params_for(wa)
        kda.run(pp, one, po, kda.alloc_workspace(pp))
        torch.cuda.synchronize()
        assert torch.equal(d["state"][idx["cache_indices"][n].item()], po["inter_ssm"][0, a - 1]), n
        assert torch.equal(d["conv_state"][idx["conv_state_indices"][n].item()], one["conv_state"][0]), n


@pytest.mark.parametrize("N,T,H,HV", [(32, 4, 16, 32), (41, 2, 1, 25), (40, 3, 8, 32)],
                         ids=["1024-units", "1025-units-uneven-conv-slices", "1280-units"])
def test_commit_both_kernel_shapes_match_oracle(N, T, H, HV):
    """The accept step at unit counts on both sides of the switch between its two kernel
    shapes (256 threads up to 1024 units, 1024 threads beyond), with the conv row split
    unevenly over the value heads (25 of them), scattered pool rows, a padding row, and
    sequences that accept nothing or every token: a bit copy, exact against the oracle, and
    rows it must not write keep their bits."""
    w = W(N, T, H, HV)
    say(f"[gpu] commit {N}x{T}x{H}x{HV} ({N * HV} units)")
    g = torch.Generator().manual_seed(21)
    cg = torch.Generator().manual_seed(22)
    slots = (N + 5, N + 3, N + 4)
    cs_idx, st_idx, in_idx = (torch.randperm(s_, generator=cg)[:N].to(torch.int32) for s_ in slots)
    st_idx[3] = -1  # padding sequence
    acc = torch.tensor([n % (T + 1) for n in range(N)], dtype=torch.int32)  # 0 (nothing) .. T
    # seeded inputs drawn on the host, then copied to the device
    inter = torch.randn((slots[2], T, HV, w.K, w.V), generator=g).cuda()
    cw = torch.randn((slots[2], T, w.C, 3), generator=g).to(w.torch_dtype).cuda()
    st = torch.randn((slots[1], HV, w.K, w.V), generator=g).cuda()
    cs = torch.randn((slots[0], w.C, 3), generator=g).to(w.torch_dtype).cuda()
    idx = {"conv_state_indices": cs_idx, "cache_indices": st_idx, "intermediate_state_indices": in_idx}
    ref = oracle.commit(acc, idx, inter, cw, st, cs, T=T)
    p = kda.params_for(w)
    # index arrays made on the fly: the descriptor keeps them alive, so the allocations that
    # follow (the accepted counts) cannot land in their memory
    pools = kda.make_pools(N, cs_idx.cuda(), st_idx.cuda(), in_idx.cuda(), *slots)
    assert [t.data_ptr() for t in pools.index_tensors] == [pools.conv_state_indices, pools.cache_indices,
                                                            pools.intermediate_state_indices]
    kda.verify_commit(p, pools, acc.cuda(), inter, cw, st, cs)
    torch.cuda.synchronize()
    assert torch.equal(st.cpu(), torch.from_numpy(ref["state"]).float())
    assert np.array_equal(bits(cs), bits(torch.from_numpy(ref["conv_state"]).to(w.torch_dtype)))


@pytest.mark.parametrize("launch", [dict(), dict(store_policy=2), dict(store_policy=2, schedule=2, max_wg_per_cu=1),
                                    dict(store_policy=2, schedule=3)],
                         ids=["auto", "device-scope-stores", "device-scope-stores-queue", "device-scope-stores-stream"])
def test_serving_loop_verify_commit_chain(launch):
    """Three rounds of verify -> commit on shared pools; each round's outputs match the
    oracle run on the pools the previous rounds left. Also with the snapshots streamed at
    device scope (on the grid and the queue): the commit and the next verify read them."""
    w = W(4, 4, 2, 4, gate="safe")
    slots = (6, 6, 5)
    pinp, idx, init = _pooled_case(w, slots, seed=11)
    ref_cs, ref_st = oracle.f64(pinp["conv_state"]), oracle.f64(pinp["state"])
    d = {k: v.cuda() for k, v in pinp.items()}
    di = {k: v.cuda() for k, v in idx.items()}
    out = {k: v.cuda() for k, v in init.items()}
    p = kda.params_for(w, **launch)
    pools = kda.make_pools(w.N, di["conv_state_indices"], di["cache_indices"], di["intermediate_state_indices"],
                           *slots)
    ws = kda.alloc_workspace(p)
    for rnd in range(3):
        fresh = synth.make_inputs(w, seed=100 + rnd)
        for k in ("mixed_qkv", "gate", "beta"):
            d[k].copy_(fresh[k])
        kda.kda_conv_verify_decode_pooled(p, pools, d["mixed_qkv"], d["conv_weight"], d["conv_state"], d["gate"],
                                          d["A_log"], d["dt_bias"], d["beta"], d["state"], out["o"],
                                          out["inter_ssm"], out["conv_window"], ws)
        acc = torch.tensor([1 + (n + rnd) % w.T for n in range(w.N)], dtype=torch.int32)
        kda.verify_commit(p, pools, acc.cuda(), out["inter_ssm"], out["conv_window"], d["state"], d["conv_state"])
        torch.cuda.synchronize()
        rin = {"mixed_qkv": fresh["mixed_qkv"], "conv_weight": pinp["conv_weight"], "gate": fresh["gate"],
               "A_log": pinp["A_log"], "dt_bias": pinp["dt_bias"], "beta": fresh["beta"],
               "conv_state": ref_cs, "state": ref_st}
        # every round writes the same pool rows, so the rows it leaves alone still hold the
        # seeded initial contents
        r = oracle.verify_pooled(rin, {**idx, **init}, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
        eo = np.abs(out["o"].float().cpu().numpy() - r["o"]).max()
        es = np.abs(out["inter_ssm"].cpu().numpy() - r["inter_ssm"]).max()
        assert eo <= TOL and es <= TOL, (rnd, eo, es)
        c = oracle.commit(acc, idx, r["inter_ssm"], r["conv_window"], ref_st, r["conv_state"], T=w.T)
        ref_cs, ref_st = c["conv_state"], c["state"]
        assert np.array_equal(bits(d["conv_state"]), bits(torch.from_numpy(ref_cs).to(w.torch_dtype))), rnd
        assert np.abs(d["state"].cpu().numpy() - ref_st).max() <= TOL, rnd


@pytest.mark.parametrize("sched", [0, 2, 3], ids=["auto", "queue", "stream"])
def test_serving_step_graph_replay_matches_eager_chain(sched):
    """One serving step (pooled verify, then commit) captured in a HIP graph and replayed for
    three rounds, each round's inputs and accepted counts copied into the captured buffers
    eagerly before its replay: after every replay the pools and outputs equal those of the
    same three rounds run eagerly, bit for bit (the commit reads the verify's snapshots
    inside one graph; on the queue and the stream each replay relies on the one before
    having zeroed the counters)."""
    w = W(24, 3, 4, 16, gate="safe")
    slots = (28, 27, 26)
    pinp, idx, init = _pooled_case(w, slots, seed=31)
    di = {k: v.cuda() for k, v in idx.items()}
    pools = kda.make_pools(w.N, di["conv_state_indices"], di["cache_indices"], di["intermediate_state_indices"],
                           *slots)
    p = kda.params_for(w, schedule=sched)
    say(f"[gpu] serving-step graph {w.name} -> {kda.select_launch(p)}")
    rounds = [synth.make_inputs(w, seed=200 + r) for r in range(3)]
    accs = [torch.tensor([(n + r) % (w.T + 1) for n in range(w.N)], dtype=torch.int32) for r in range(3)]

    def fresh_state():
        d = {k: v.cuda() for k, v in pinp.items()}
        return d, {k: v.cuda() for k, v in init.items()}, torch.zeros(w.N, dtype=torch.int32, device="cuda")

    def step(d, out, acc, ws):
        kda.kda_conv_verify_decode_pooled(p, pools, d["mixed_qkv"], d["conv_weight"], d["conv_state"], d["gate"],
                                          d["A_log"], d["dt_bias"], d["beta"], d["state"], out["o"],
                                          out["inter_ssm"], out["conv_window"], ws)
        kda.verify_commit(p, pools, acc, out["inter_ssm"], out["conv_window"], d["state"], d["conv_state"])

    def load_round(d, acc, r):
        for k in ("mixed_qkv", "gate", "beta"):
            d[k].copy_(rounds[r][k])
        acc.copy_(accs[r])

    def snap(d, out):
        return {**{k: v.clone() for k, v in out.items()}, "state": d["state"].clone(),
                "conv_state": d["conv_state"].clone()}

    # eager chain
    d, out, acc = fresh_state()
    ws = kda.alloc_workspace(p)
    eager = []
    for r in range(3):
        load_round(d, acc, r)
        step(d, out, acc, ws)
        torch.cuda.synchronize()
        eager.append(snap(d, out))
    # captured step, replayed over the same rounds from the same starting pools
    d, out, acc = fresh_state()
    ws = kda.alloc_workspace(p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        load_round(d, acc, 0)
        step(d, out, acc, ws)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    d, out, acc = fresh_state()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(d, out, acc, ws)
    for r in range(3):
        load_round(d, acc, r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snap(d, out)
        for k in got:
            assert torch.equal(got[k], eager[r][k]), (r, k)
    assert int(ws.count_nonzero().item()) == 0


def test_pool_argument_errors():
    w = W(3, 2, 1, 2)
    p = kda.params_for(w)
    inp = {k: v.cuda() for k, v in synth.make_inputs(w).items()}
    out = kda.alloc_outputs(w)
    ws = kda.alloc_workspace(p)

    def call(pools):
        kda.kda_conv_verify_decode_pooled(p, pools, inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"],
                                          inp["gate"], inp["A_log"], inp["dt_bias"], inp["beta"], inp["state"],
                                          out["o"], out["inter_ssm"], out["conv_window"], ws)

    bad = kda.make_pools(w.N)
    bad.state_slots = 0
    with pytest.raises(Exception):
        call(bad)
    lib = kda.load()
    import ctypes

    ptrs = [t.data_ptr() for t in (inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"], inp["gate"],
                                   inp["A_log"], inp["dt_bias"], inp["beta"], inp["state"], out["o"],
                                   out["inter_ssm"], out["conv_window"], ws)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def raw(pd):
        return lib.kda_conv_verify_decode_pooled(ctypes.byref(p), ctypes.byref(pd), *[ctypes.c_void_p(x) for x in ptrs],
                                                 ws.numel(), stream)

    pd = kda.make_pools(w.N)
    pd.state_slots = 0
    assert raw(pd) == -2
    pd = kda.make_pools(w.N)
    pd.intermediate_slots = w.N - 1  # identity rows need N slots
    assert raw(pd) == -2
    idx = torch.zeros(w.N + 1, dtype=torch.int32, device="cuda")
    pd = kda.make_pools(w.N)
    pd.cache_indices = idx.data_ptr() + 2  # misaligned int32 array
    assert raw(pd) == -4
    pd = kda.make_pools(w.N)
    pd.conv_state_indices = out["o"].data_ptr()  # index array inside a written buffer
    assert raw(pd) == -7


@pytest.mark.parametrize("w", [W(4, 4, 2, 4, gate="safe"), W(64, 4, 16, 32)], ids=["grid", "stream"])
def test_commit_free_chain_equals_verify_commit_chain(w):
    """A batch whose sequences all advance every step can skip the accept step: the next
    verify takes its state rows from the previous step's inter_ssm viewed as N*T state rows
    (row n*T + a_n - 1, the accepted token's snapshot) and its conv-cache rows from the
    previous conv_window viewed the same way, and writes its own snapshots to a second set
    of buffers (the two alternate). Over three steps with varying accepted counts this gives
    the same bits as verify -> commit on a state and a conv-cache pool: o, inter_ssm and
    conv_window of every step, and the state and conv cache each chain holds at the end.
    The 64-sequence case runs on the stream (2048 units at T = 4)."""
    p = kda.params_for(w)
    ws = kda.alloc_workspace(p)
    d = {k: v.cuda() for k, v in synth.make_inputs(w).items()}
    ident = kda.make_pools(w.N)
    st_a, cs_a = d["state"].clone(), d["conv_state"].clone()  # chain A: pools the commit updates
    out_a = kda.alloc_outputs(w)
    bufs = [kda.alloc_outputs(w), kda.alloc_outputs(w)]  # chain B: alternating snapshot sets
    st_b, cs_b = d["state"].clone(), d["conv_state"].clone()
    NT = w.N * w.T
    seq = torch.arange(w.N, dtype=torch.int32, device="cuda")
    acc = None
    for step in range(3):
        fresh = synth.make_inputs(w, seed=300 + step)
        for k in ("mixed_qkv", "gate", "beta"):
            d[k].copy_(fresh[k])
        say(f"[gpu] commit-free chain {w.name} step {step}")
        kda.kda_conv_verify_decode_pooled(p, ident, d["mixed_qkv"], d["conv_weight"], cs_a, d["gate"], d["A_log"],
                                          d["dt_bias"], d["beta"], st_a, out_a["o"], out_a["inter_ssm"],
                                          out_a["conv_window"], ws)
        cur = bufs[step % 2]
        if acc is None:
            pools, cs_src, st_src = ident, cs_b, st_b
        else:
            prev = bufs[(step - 1) % 2]
            rows = seq * w.T + acc - 1
            pools = kda.make_pools(w.N, rows, rows, None, NT, NT, w.N)
            cs_src, st_src = prev["conv_window"].view(NT, w.C, 3), prev["inter_ssm"].view(NT, w.HV, w.K, w.V)
        kda.kda_conv_verify_decode_pooled(p, pools, d["mixed_qkv"], d["conv_weight"], cs_src, d["gate"], d["A_log"],
                                          d["dt_bias"], d["beta"], st_src, cur["o"], cur["inter_ssm"],
                                          cur["conv_window"], ws)
        acc = torch.tensor([1 + (3 * n + step) % w.T for n in range(w.N)], dtype=torch.int32, device="cuda")
        kda.verify_commit(p, ident, acc, out_a["inter_ssm"], out_a["conv_window"], st_a, cs_a)
        torch.cuda.synchronize()
        for k in ("o", "inter_ssm", "conv_window"):
            assert np.array_equal(bits(out_a[k]), bits(cur[k])), (step, k)
    last = bufs[2 % 2]
    pick = (seq.long(), (acc - 1).long())
    assert np.array_equal(bits(st_a), bits(last["inter_ssm"][pick])), "state after the last step"
    assert np.array_equal(bits(cs_a), bits(last["conv_window"][pick])), "conv cache after the last step"


@pytest.mark.parametrize("w", [W(6, 4, 2, 4, gate="safe"), W(64, 4, 16, 32)], ids=["grid", "stream"])
def test_commit_free_step_graph_replay_matches_eager(w):
    """The serving step without the accept step, captured as two HIP graphs (one per
    direction between the two alternating snapshot sets) and replayed over four rounds, each
    round's inputs and accepted-row indices copied into the captured buffers eagerly before
    its replay: after every replay both snapshot sets equal those of the same rounds run
    eagerly, bit for bit, and the workspace counters are back to zero."""
    p = kda.params_for(w)
    NT = w.N * w.T
    base = synth.make_inputs(w)
    rounds = [synth.make_inputs(w, seed=400 + r) for r in range(4)]
    accs = [torch.tensor([1 + (5 * n + r) % w.T for n in range(w.N)], dtype=torch.int32) for r in range(4)]
    say(f"[gpu] commit-free graph {w.name} -> {kda.select_launch(p)}")

    def setup():
        d = {k: v.cuda() for k, v in base.items()}
        bufs = [kda.alloc_outputs(w), kda.alloc_outputs(w)]
        rows = torch.zeros(w.N, dtype=torch.int32, device="cuda")
        ws = kda.alloc_workspace(p)
        kda.run(p, d, bufs[1], ws)  # the first step, from the initial state and conv cache
        torch.cuda.synchronize()
        return d, bufs, rows, ws

    def load_round(d, rows, r):
        for k in ("mixed_qkv", "gate", "beta"):
            d[k].copy_(rounds[r][k])
        rows.copy_(torch.arange(w.N, dtype=torch.int32) * w.T + accs[r] - 1)

    def step(d, bufs, rows, ws, src):
        prev, cur = bufs[src], bufs[1 - src]
        pools = kda.make_pools(w.N, rows, rows, None, NT, NT, w.N)
        kda.kda_conv_verify_decode_pooled(p, pools, d["mixed_qkv"], d["conv_weight"],
                                          prev["conv_window"].view(NT, w.C, 3), d["gate"], d["A_log"], d["dt_bias"],
                                          d["beta"], prev["inter_ssm"].view(NT, w.HV, w.K, w.V), cur["o"],
                                          cur["inter_ssm"], cur["conv_window"], ws)

    def snap(bufs):
        return [{k: v.clone() for k, v in b.items()} for b in bufs]

    d, bufs, rows, ws = setup()
    eager = []
    for r in range(4):  # round r reads set (r + 1) % 2 and writes the other
        load_round(d, rows, r)
        step(d, bufs, rows, ws, (r + 1) % 2)
        torch.cuda.synchronize()
        eager.append(snap(bufs))

    d, bufs, rows, ws = setup()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        load_round(d, rows, 0)
        step(d, bufs, rows, ws, 1)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    d, bufs, rows, ws = setup()
    graphs = [torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()]
    for src in (0, 1):
        with torch.cuda.graph(graphs[src]):
            step(d, bufs, rows, ws, src)
    for r in range(4):
        load_round(d, rows, r)
        torch.cuda.synchronize()
        graphs[(r + 1) % 2].replay()
        torch.cuda.synchronize()
        got = snap(bufs)
        for i in (0, 1):
            for k in got[i]:
                assert torch.equal(got[i][k], eager[r][i][k]), (r, i, k)
    assert int(ws.count_nonzero().item()) == 0


def _random_pooled(seed=13, draws=30):
    """Seeded random pooled cases: shape, pool sizes, padding entries and a schedule."""
    rng, out = random.Random(seed), []
    for i in range(draws):
        K = rng.choice([16, 64, 128, 128])
        H = rng.choice([1, 2, 4])
        g = rng.choice([1, 2, 3])
        T = rng.choice([1, 2, 3, 4, 6, 8])
        N = rng.randint(1, 24)
        dtype = rng.choice(["bf16", "bf16", "f32"])
        gate = rng.choice(["softplus", "safe"])
        w = W(N, T, H, H * g, K=K, V=K, dtype=dtype, gate=gate, seed=900 + i)
        slots = tuple(N + rng.randint(0, 8) for _ in range(3))
        pad = tuple(sorted(rng.sample(range(N), rng.randint(0, min(3, N - 1))))) if N > 1 else ()
        kw = {}
        if K == 128:
            kw = rng.choice([{}, dict(schedule=2), dict(schedule=3), dict(schedule=3, prefetch=1),
                             dict(schedule=1, tile_columns=32)])
        out.append((w, slots, pad, kw))
    return out


RANDOM_POOLED = _random_pooled()


@pytest.mark.parametrize("w,slots,pad,kw", RANDOM_POOLED,
                         ids=[f"{c[0].name}-{c[0].dtype}-{c[0].gate}-slots{'x'.join(map(str, c[1]))}-pad{len(c[2])}"
                              f"-{'-'.join(f'{k}{v}' for k, v in c[3].items()) or 'auto'}" for c in RANDOM_POOLED])
def test_random_pooled_shapes_match_oracle(w, slots, pad, kw):
    """Seeded random shapes on pools larger than the batch, rows picked at random, up to
    three padding entries, on the AUTO launch, the queue, the stream (either prefetch point)
    or 32-column grid tiles; every output against the oracle's pooled step (padding rows of
    o left as they were, conv bits exact)."""
    pinp, idx, init = _pooled_case(w, slots, seed=w.seed, pad=pad)
    got, *_ = _run_pooled(w, pinp, idx, init, **kw)
    ref = oracle.verify_pooled(pinp, {**idx, **init}, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    _compare(w, got, ref)
