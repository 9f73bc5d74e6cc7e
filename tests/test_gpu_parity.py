"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

conv_window and conv_state must match bit for bit; o and inter_ssm within max-abs
2e-3 (bf16 or fp32 inputs, fp32 state and arithmetic). Every output buffer is
filled with NaN first, so an element the kernel forgets to write fails the check.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request),
Tests & Accuracy: bit-exact conv window / cache, tolerance on o and the snapshots,
both gate forms, H == HV and GVA, several T, both variants.
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches, assert_matches_all, run_gpu, say, slice_inputs

pytestmark = pytest.mark.gpu

S, L, A = kda.VARIANT_SMALL, kda.VARIANT_LARGE, kda.VARIANT_AUTO


def W(N, T, H, HV, K, V, dtype="bf16", gate="softplus", seed=7):
    return synth.Workload(f"case{N}x{T}x{H}x{HV}x{K}", N=N, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, gate=gate,
                          seed=seed)


def test_tiny_workload_both_gates():
    for gate in ("softplus", "safe"):
        w = synth.WORKLOADS["tiny"].with_(gate=gate)
        inp = synth.make_inputs(w)
        got = run_gpu(w, inp)
        assert_matches(w, got, oracle.verify_workload(w, inp), what=f"tiny {gate}")


# Small shapes the oracle finishes in well under a second: several WGs and V-tiles,
# odd N, every TMAX tier (T = 1, 2, 3, 5, 8, 9, 16), GVA with g = 2, 3, 4, both
# variants, both gate forms, bf16 and fp32 inputs, K = V = 16, 64, 128.
CASES = [
    (W(3, 1, 2, 2, 128, 128), L),
    (W(3, 1, 2, 2, 128, 128, gate="safe"), S),
    (W(3, 2, 2, 4, 128, 128, gate="safe"), S),
    (W(3, 2, 2, 4, 128, 128), L),
    (W(2, 3, 1, 4, 128, 128), A),
    (W(5, 5, 2, 2, 128, 128, dtype="f32", gate="safe"), L),
    (W(5, 5, 2, 2, 128, 128, dtype="f32"), S),
    (W(2, 8, 2, 2, 128, 128), S),
    (W(2, 8, 1, 3, 128, 128, gate="safe"), L),
    (W(1, 9, 1, 1, 128, 128), S),
    (W(1, 16, 1, 2, 128, 128, gate="safe"), L),
    (W(2, 16, 1, 1, 128, 128, dtype="f32"), S),
    (W(3, 4, 2, 2, 64, 64), L),
    (W(3, 4, 2, 4, 64, 64, gate="safe"), S),
    (W(3, 7, 1, 2, 64, 64, dtype="f32"), A),
    (W(4, 3, 1, 3, 16, 16, dtype="f32", gate="safe"), A),
    (W(2, 6, 2, 6, 16, 16), A),
    (W(1, 16, 1, 1, 16, 16, dtype="f32"), A),
]


@pytest.mark.parametrize("w,variant", CASES, ids=[f"{w.name}-{w.dtype}-{w.gate}-v{v}" for w, v in CASES])
def test_small_shapes(w, variant):
    inp = synth.make_inputs(w)
    got = run_gpu(w, inp, variant)
    assert_matches(w, got, oracle.verify_workload(w, inp), what=w.name)


@pytest.mark.parametrize("name", ["small_batch", "gva", "large_batch", "max_bandwidth"])
def test_workload_full_size(name):
    """Each named workload at its full size in the launch configuration the benchmark
    times (AUTO): every sequence's o, inter_ssm, conv_window and rolled conv_state against
    the oracle, which runs on all host threads in slices of four sequences while the GPU
    outputs come back slice by slice (max_bandwidth's inter_ssm is 16 GiB)."""
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    got = run_gpu(w, inp, A)
    say(f"[gpu] {name}: oracle on all {w.N} sequences")
    err = assert_matches_all(w, inp, got, what=name)
    say(f"{name}: all {w.N} sequences, max-abs o={err['o']:.2e} inter_ssm={err['inter_ssm']:.2e}")


def test_variants_bit_identical():
    """SMALL and LARGE share one K-sum tree, so they agree bit for bit (K = V = 128)."""
    for w in (W(4, 4, 2, 4, 128, 128, gate="safe"), W(3, 8, 2, 2, 128, 128, dtype="f32")):
        inp = synth.make_inputs(w)
        a = run_gpu(w, inp, S)
        b = run_gpu(w, inp, L)
        for k in ("o", "inter_ssm", "conv_window", "conv_state"):
            assert torch.equal(a[k].view(torch.int16 if a[k].element_size() == 2 else torch.int32),
                               b[k].view(torch.int16 if b[k].element_size() == 2 else torch.int32)), k


def _chained(w, inp, variant):
    """T one-token calls, each fed the previous snapshot and rolled conv cache."""
    w1 = w.with_(T=1)
    cs, st = inp["conv_state"], inp["state"]
    outs = []
    for t in range(w.T):
        step = dict(inp)
        step["mixed_qkv"] = inp["mixed_qkv"][:, t:t + 1].contiguous()
        step["gate"] = inp["gate"][:, t:t + 1].contiguous()
        step["beta"] = inp["beta"][:, t:t + 1].contiguous()
        step["conv_state"], step["state"] = cs, st
        o = run_gpu(w1, step, variant)
        outs.append(o)
        cs, st = o["conv_state"], o["inter_ssm"][:, 0].contiguous()
    return outs


@pytest.mark.parametrize("w,variant", [(W(3, 5, 2, 4, 128, 128, gate="safe"), A), (W(2, 4, 1, 1, 16, 16, dtype="f32"), A),
                                       (W(2, 6, 2, 2, 128, 128), S)])
def test_t_token_verify_equals_chained_decode(w, variant):
    """A T-token verify equals T chained one-token calls. Each token runs the same
    fp32 operations on the same bits in both, so the match is exact."""
    inp = {k: v.cuda() for k, v in synth.make_inputs(w).items()}
    full = run_gpu(w, {k: v.clone() for k, v in inp.items()}, variant)
    outs = _chained(w, inp, variant)
    for t, o in enumerate(outs):
        assert torch.equal(o["inter_ssm"][:, 0], full["inter_ssm"][:, t]), t
        assert torch.equal(o["o"][:, 0], full["o"][:, t]), t
        assert torch.equal(o["conv_window"][:, 0], full["conv_window"][:, t]), t
    assert torch.equal(outs[-1]["conv_state"], full["conv_state"])


def test_max_bandwidth_t_token_vs_chained_full_size():
    """The Max bandwidth workload (N=512, T=8, H=16, HV=64, K=V=128): T-token verify
    against 8 chained one-token calls, compared on the GPU."""
    w = synth.WORKLOADS["max_bandwidth"]
    inp = {k: v.cuda() for k, v in synth.make_inputs(w).items()}
    full = run_gpu(w, {k: v.clone() for k, v in inp.items()}, A, poison=False)
    w1 = w.with_(T=1)
    cs, st = inp["conv_state"], inp["state"]
    for t in range(w.T):
        step = dict(inp)
        step["mixed_qkv"] = inp["mixed_qkv"][:, t:t + 1].contiguous()
        step["gate"] = inp["gate"][:, t:t + 1].contiguous()
        step["beta"] = inp["beta"][:, t:t + 1].contiguous()
        step["conv_state"], step["state"] = cs, st
        o = run_gpu(w1, step, A, poison=False)
        assert torch.equal(o["inter_ssm"][:, 0], full["inter_ssm"][:, t]), t
        assert torch.equal(o["o"][:, 0], full["o"][:, t]), t
        cs, st = o["conv_state"], o["inter_ssm"][:, 0].contiguous()
        del o
    assert torch.equal(cs, full["conv_state"])


def _expand_gva(w, inp):
    H, HV, K, g = w.H, w.HV, w.K, w.HV // w.H
    qk_idx = []
    for blk in range(2):
        for hv in range(HV):
            h = hv // g
            qk_idx.extend(range(blk * H * K + h * K, blk * H * K + (h + 1) * K))
    idx = torch.tensor(qk_idx + list(range(2 * H * K, w.C)))
    e = dict(inp)
    e["mixed_qkv"] = inp["mixed_qkv"][:, :, idx].contiguous()
    e["conv_weight"] = inp["conv_weight"][idx].contiguous()
    e["conv_state"] = inp["conv_state"][:, idx].contiguous()
    return w.with_(H=HV), e, idx


@pytest.mark.parametrize("w,variant", [(W(3, 4, 2, 4, 128, 128), S), (W(2, 3, 1, 4, 128, 128, gate="safe"), L),
                                       (W(2, 5, 1, 3, 16, 16, dtype="f32"), A)])
def test_gva_equals_head_repetition(w, variant):
    """HV > H gives exactly what H' = HV with each q/k head repeated gives."""
    inp = synth.make_inputs(w)
    we, ie, idx = _expand_gva(w, inp)
    a = run_gpu(w, inp, variant)
    b = run_gpu(we, ie, variant)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["inter_ssm"], b["inter_ssm"])
    assert torch.equal(a["conv_window"][:, :, idx.cuda()], b["conv_window"])
    assert torch.equal(a["conv_state"][:, idx.cuda()], b["conv_state"])


def test_beta0_no_decay_leaves_state():
    """beta = 0 and zero log-decay: every snapshot equals the state bit for bit."""
    for gate in ("softplus", "safe"):
        w = W(3, 4, 2, 4, 128, 128, gate=gate)
        inp = synth.make_inputs(w)
        inp["beta"] = torch.full_like(inp["beta"], float("-inf"))
        inp["gate"] = torch.full_like(inp["gate"], float("-inf"))
        got = run_gpu(w, inp)
        for t in range(w.T):
            assert torch.equal(got["inter_ssm"][:, t].cpu(), inp["state"]), (gate, t)


def test_identity_taps_give_silu():
    """Identity conv taps: conv + SiLU is SiLU(x_t); with beta = 0, no decay and an
    identity state (K = V), o_t is the normalised, scaled q_t."""
    w = W(2, 3, 2, 2, 16, 16, dtype="f32")
    inp = synth.make_inputs(w)
    inp["conv_weight"] = torch.tensor([0.0, 0.0, 0.0, 1.0]).repeat(w.C, 1)
    inp["beta"] = torch.full_like(inp["beta"], float("-inf"))
    inp["gate"] = torch.full_like(inp["gate"], float("-inf"))
    inp["state"] = torch.eye(16).expand(w.N, w.HV, 16, 16).contiguous()
    got = run_gpu(w, inp)
    q = torch.nn.functional.silu(inp["mixed_qkv"][..., : w.H * w.K].double()).reshape(w.N, w.T, w.H, w.K)
    q = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6) * w.K ** -0.5
    np.testing.assert_allclose(got["o"].cpu().double().numpy(), q.numpy(), atol=1e-5)


def test_extreme_gate_and_beta_stay_finite():
    """Gate inputs far past the softplus threshold: no overflow turned into NaN."""
    w = W(2, 4, 2, 2, 128, 128, gate="softplus")
    inp = synth.make_inputs(w)
    vals = torch.tensor([1e4, -1e4, 3e38, -3e38, 88.0, 30.0])
    inp["gate"] = vals.repeat(inp["gate"].numel() // 6 + 1)[: inp["gate"].numel()].reshape(inp["gate"].shape).to(torch.bfloat16)
    inp["beta"] = torch.full_like(inp["beta"], 1e4)
    for gate in ("softplus", "safe"):
        ww = w.with_(gate=gate)
        got = run_gpu(ww, inp)
        assert_matches(ww, got, oracle.verify_workload(ww, inp), what=f"extreme {gate}")


def test_zero_q_k_channels():
    w = W(2, 3, 2, 2, 128, 128)
    inp = synth.make_inputs(w)
    inp["conv_weight"][: 2 * w.H * w.K] = 0
    got = run_gpu(w, inp)
    assert_matches(w, got, oracle.verify_workload(w, inp), what="zero q/k")
    assert torch.count_nonzero(got["o"]) == 0


@pytest.mark.parametrize("w", [W(64, 4, 16, 32, 128, 128, gate="safe"),   # 2048 units at T = 4, device-scope streaming stores
                               W(16, 4, 8, 16, 128, 128),                  # 256 units, T HV = 64: streaming stores
                               W(32, 8, 16, 32, 128, 128, gate="safe")])   # T = 8, shared q/k heads, 1024 units: streaming
def test_every_tile_shape_bit_identical(w):
    """SMALL (32-column WGs) and LARGE (whole-V WGs) with the store policy dispatch picks for
    the shape give the same bits; every sequence is also checked against the oracle."""
    inp = synth.make_inputs(w)
    a = run_gpu(w, inp, S)
    b = run_gpu(w, inp, L)
    for k in ("o", "inter_ssm", "conv_window", "conv_state"):
        assert torch.equal(a[k], b[k]), k
    assert_matches_all(w, inp, a, what=f"tile shapes {w.name}")


@pytest.mark.parametrize("w", [W(5, 3, 2, 4, 128, 128, gate="safe"),     # up to 4 tokens per WG
                               W(6, 8, 2, 4, 128, 128),                  # up to 8
                               W(3, 12, 1, 2, 128, 128, gate="safe")])   # up to 16
def test_explicit_tile_and_store_overrides_bit_identical(w):
    """Every tile width (32, 64, 128 columns per WG), both snapshot store policies, the
    workgroups-per-CU caps, both schedules and both unit orders give the same bits, for
    each token-count template; one of them
    is checked against the oracle. (The device-scope store is inline assembly: a missing
    wait after it once let later VALU writes reach memory in place of the snapshot.)"""
    inp = synth.make_inputs(w)
    outs = []
    for tile in (32, 64, 128):
        for pol in (1, 2):
            outs.append(run_gpu(w, inp, A, tile_columns=tile, store_policy=pol))
    for tile, occ in ((32, 1), (64, 2), (128, 4), (64, 6), (128, 1)):  # per-CU caps: scheduling only
        outs.append(run_gpu(w, inp, A, tile_columns=tile, max_wg_per_cu=occ))
    for groups in (2, 4):  # whole-V workgroups split into column groups of 4 waves
        for pol in (1, 2):
            outs.append(run_gpu(w, inp, A, tile_columns=128, column_groups=groups, store_policy=pol, max_wg_per_cu=1))
    for groups, pol, occ in ((1, 1, 1), (2, 2, 1), (4, 1, 8)):  # the queue schedule
        outs.append(run_gpu(w, inp, A, tile_columns=128, column_groups=groups, store_policy=pol, max_wg_per_cu=occ,
                            schedule=2))
    for tile, order in ((128, 1), (128, 2), (32, 2), (64, 1)):  # unit orders of the grid
        outs.append(run_gpu(w, inp, A, tile_columns=tile, unit_order=order))
    for o in outs[1:]:
        for k in ("o", "inter_ssm", "conv_window", "conv_state"):
            assert torch.equal(o[k], outs[0][k]), k
    assert_matches(w, outs[0], oracle.verify_workload(w, inp), what="overrides")
