"""Pins of the float64 CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a special case that
reduces to a textbook/library routine (torch.nn.functional.conv1d, silu, softplus,
normalize; numpy matrix products), an invariant of the method (chained decode, GVA as
head repetition, beta = 0 / alpha = 1), or brute force on tiny shapes. Chosen so that a
plausible slip in the oracle (reversed taps, an off-by-one window, a dropped scale or
bias, a wrong sign, a transposed operand, a wrong head map) fails at least one.

Source page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linear_attention_decode_kda_amd import synth

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _rng(seed):
    return np.random.default_rng(seed)


def _ext_seq(x, s):
    """Extended raw sequence [N, C, 3+T]: the cached three tokens, then the new ones."""
    return np.concatenate([s, np.transpose(x, (0, 2, 1))], axis=2)


# ---------------------------------------------------------------- conv window / conv_state
@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_conv_roll_is_shift_register(T):
    """PR#107 description: conv_state holds the three most recent raw tokens; the per-token
    window is the cache that a rollback to token t restores. Values encode (n, tau, c),
    so any misplaced element is seen."""
    N, C = 3, 7
    x = np.zeros((N, T, C))
    s = np.zeros((N, C, 3))
    code = lambda n, tau, c: 10000 * n + 100 * tau + c + 1  # noqa: E731
    for n in range(N):
        for c in range(C):
            for tau in range(3):
                s[n, c, tau] = code(n, tau, c)
            for t in range(T):
                x[n, t, c] = code(n, t + 3, c)
    cw, cs = oracle.conv_roll(x, s)
    for n in range(N):
        for c in range(C):
            for t in range(T):
                assert list(cw[n, t, c]) == [code(n, t + 1 + j, c) for j in range(3)]
            assert list(cs[n, c]) == [code(n, T + j, c) for j in range(3)]
    # the same, written with numpy sliding windows over the extended sequence
    E = _ext_seq(x, s)
    win = np.lib.stride_tricks.sliding_window_view(E, 3, axis=2)  # [N, C, T+1, 3]
    np.testing.assert_array_equal(cw, np.transpose(win[:, :, 1:T + 1, :], (0, 2, 1, 3)))
    np.testing.assert_array_equal(cs, win[:, :, T, :])
    # last window row equals the rolled cache
    np.testing.assert_array_equal(cw[:, T - 1], cs)


def test_conv_roll_short_T_literal():
    """T = 1 and T = 2 keep 2 and 1 old cache entries (any T >= 1 is allowed, PR#107 commit 1)."""
    s = np.array([[[1.0, 2.0, 3.0]]])
    cw, cs = oracle.conv_roll(np.array([[[4.0]]]), s)
    assert cs.tolist() == [[[2.0, 3.0, 4.0]]] and cw.tolist() == [[[[2.0, 3.0, 4.0]]]]
    cw, cs = oracle.conv_roll(np.array([[[4.0], [5.0]]]), s)
    assert cs.tolist() == [[[3.0, 4.0, 5.0]]]
    assert cw.tolist() == [[[[2.0, 3.0, 4.0]], [[3.0, 4.0, 5.0]]]]


# ---------------------------------------------------------------- conv + SiLU
def test_identity_taps_reduce_to_silu():
    """Taps [0, 0, 0, 1]: the causal conv is the identity on the current token."""
    r = _rng(1)
    N, T, C = 2, 4, 6
    x, s = r.normal(size=(N, T, C)), r.normal(size=(N, C, 3))
    w = np.tile([0.0, 0.0, 0.0, 1.0], (C, 1))
    act = oracle.conv_silu(x, w, s)
    np.testing.assert_allclose(act, F.silu(torch.from_numpy(x)).numpy(), rtol=0, atol=1e-15)


@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_unit_tap_selects_window_element(j):
    """A single unit tap at position j gives SiLU(e[t + j]); j = 3 is the newest token."""
    r = _rng(2 + j)
    N, T, C = 2, 5, 4
    x, s = r.normal(size=(N, T, C)), r.normal(size=(N, C, 3))
    w = np.zeros((C, 4))
    w[:, j] = 1.0
    E = _ext_seq(x, s)  # [N, C, T+3]
    want = F.silu(torch.from_numpy(E[:, :, j:j + T])).numpy().transpose(0, 2, 1)
    np.testing.assert_allclose(oracle.conv_silu(x, w, s), want, rtol=0, atol=1e-15)


def test_conv_matches_torch_conv1d():
    """Library routine: depthwise F.conv1d (cross-correlation) over the cache-prefixed sequence."""
    r = _rng(7)
    N, T, C = 3, 6, 10
    x, s, w = r.normal(size=(N, T, C)), r.normal(size=(N, C, 3)), r.normal(size=(C, 4)) * 0.5
    E = torch.from_numpy(_ext_seq(x, s))
    y = F.conv1d(E, torch.from_numpy(w).unsqueeze(1), groups=C)  # [N, C, T]
    want = F.silu(y).numpy().transpose(0, 2, 1)
    np.testing.assert_allclose(oracle.conv_silu(x, w, s), want, rtol=1e-13, atol=1e-14)


def test_silu_sigmoid_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(-math.inf) == 0.0 and oracle.sigmoid(math.inf) == 1.0
    for y in np.linspace(-30, 30, 61):
        assert oracle.silu(y) == pytest.approx(F.silu(torch.tensor(y, dtype=torch.float64)).item(), rel=1e-14, abs=1e-300)
        assert oracle.sigmoid(y) == pytest.approx(torch.sigmoid(torch.tensor(y, dtype=torch.float64)).item(), rel=1e-14)
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)


# ---------------------------------------------------------------- l2norm
def test_l2norm_closed_form():
    r = _rng(3)
    x = r.normal(size=128)
    eps, scale = 1e-6, 128 ** -0.5
    out = oracle.l2norm(x, eps=eps, scale=scale)
    s = float(np.sum(x * x))
    assert float(np.sum(out * out)) == pytest.approx(scale * scale * s / (s + eps), rel=1e-13)
    # direction preserved with a positive factor
    np.testing.assert_allclose(out / np.linalg.norm(out), x / np.linalg.norm(x), atol=1e-15)
    # eps = 0 reduces to the library normalize
    np.testing.assert_allclose(oracle.l2norm(x, eps=0.0), F.normalize(torch.from_numpy(x), dim=0).numpy(), atol=1e-15)
    # an all-zero head is 0, not NaN
    assert np.all(oracle.l2norm(np.zeros(16), eps=eps) == 0.0)


# ---------------------------------------------------------------- gate and beta
def test_softplus_matches_library_and_threshold_branch():
    """torch's softplus has the same beta/threshold semantics (linear above beta*x > threshold)."""
    for b in (1.0, 0.5, 2.0):
        for thr in (20.0, 5.0):
            for x in np.concatenate([np.linspace(-40, 40, 81), [thr / b, thr / b + 1e-9]]):
                want = F.softplus(torch.tensor(x, dtype=torch.float64), beta=b, threshold=thr).item()
                assert oracle.softplus(x, b, thr) == pytest.approx(want, rel=1e-14, abs=1e-300)
    # past the threshold the value is x itself; no overflow even far past it (PR#107 review)
    assert oracle.softplus(1e4) == 1e4 and oracle.softplus(1e308) == 1e308
    assert oracle.softplus(-1e4) == 0.0


@pytest.mark.parametrize("mode", [oracle.GATE_SOFTPLUS, oracle.GATE_SAFE])
def test_log_decay_special_points(mode):
    lb = -5.0
    # gamma = -inf -> no decay in both forms
    assert oracle.log_decay(mode, -math.inf, 0.0, 0.3, lb) == 0.0
    # large inputs stay finite (no NaN from a formed-then-discarded exponential)
    for g in (1e4, -1e4, 3e38):
        assert math.isfinite(oracle.log_decay(mode, g, 0.0, 0.7, lb))
    # alpha = exp(log-decay) lies in (0, 1]
    for g in np.linspace(-8, 8, 33):
        ld = oracle.log_decay(mode, g, 0.05, 0.4, lb)
        assert ld <= 0.0 and math.exp(ld) <= 1.0
        if mode == oracle.GATE_SAFE:
            assert lb <= ld


def test_log_decay_softplus_form():
    # A_log = -inf: exp(A_log) = 0 -> no decay
    assert oracle.log_decay(0, 1.3, 0.0, -math.inf) == 0.0
    # gamma = 0 (dt_bias cancels g): -exp(A) * ln 2
    assert oracle.log_decay(0, 0.25, -0.25, 0.0) == pytest.approx(-math.log(2.0), rel=1e-15)
    assert oracle.log_decay(0, 0.25, -0.25, math.log(2.0)) == pytest.approx(-2 * math.log(2.0), rel=1e-15)
    # linear tail: beta*gamma > threshold -> exactly -exp(A) * gamma
    assert oracle.log_decay(0, 30.0, 0.5, 0.0) == -30.5
    # softplus_beta scales inside and outside the log
    assert oracle.log_decay(0, 1.0, 0.0, 0.0, softplus_beta=2.0) == pytest.approx(-math.log1p(math.exp(2.0)) / 2.0, rel=1e-15)


def test_log_decay_safe_form():
    lb = -5.0
    # gamma = 0 -> lb * sigmoid(0) = lb / 2
    assert oracle.log_decay(1, 0.1, -0.1, 0.9, lb) == pytest.approx(lb / 2, rel=1e-15)
    # gamma -> +inf saturates at the lower bound
    assert oracle.log_decay(1, 1e4, 0.0, 0.0, lb) == lb
    # sigmoid(exp(A) * gamma) with exp(A) = 2, gamma = ln(3)/2 -> 3/4
    assert oracle.log_decay(1, math.log(3.0) / 2, 0.0, math.log(2.0), lb) == pytest.approx(0.75 * lb, rel=1e-14)


# ---------------------------------------------------------------- delta rule
@pytest.mark.parametrize("K,V", [(4, 4), (3, 5), (6, 2)])
def test_delta_step_bruteforce_dense(K, V):
    """Dense matrix form S' = (I - b k k^T) Diag(a) S + b k v^T, o = S'^T q. K != V catches transposes."""
    r = _rng(10 * K + V)
    S = r.normal(size=(K, V))
    a, k, v, q = r.uniform(0.1, 1.0, size=K), r.normal(size=K), r.normal(size=V), r.normal(size=K)
    b = 0.37
    Sn, o = oracle.delta_step(S, a, k, v, b, q)
    want = (np.eye(K) - b * np.outer(k, k)) @ np.diag(a) @ S + b * np.outer(k, v)
    np.testing.assert_allclose(Sn, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o, want.T @ q, rtol=1e-13, atol=1e-13)


def test_delta_rule_write_property():
    """alpha = 1, beta = 1, unit k: after the write the state maps k exactly to v."""
    r = _rng(5)
    K, V = 8, 5
    S = r.normal(size=(K, V))
    k = r.normal(size=K)
    k /= np.linalg.norm(k)
    v = r.normal(size=V)
    Sn, _ = oracle.delta_step(S, np.ones(K), k, v, 1.0, np.zeros(K))
    np.testing.assert_allclose(Sn.T @ k, v, atol=1e-13)
    # general beta: S'^T k = (1 - b) S^T k + b v for unit k
    Sn, _ = oracle.delta_step(S, np.ones(K), k, v, 0.3, np.zeros(K))
    np.testing.assert_allclose(Sn.T @ k, 0.7 * (S.T @ k) + 0.3 * v, atol=1e-13)


# ---------------------------------------------------------------- whole verify step
def _small_inputs(N=2, T=3, H=2, HV=2, K=8, V=8, seed=0, dtype="f32", gate="softplus"):
    w = synth.Workload("t", N=N, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, gate=gate, seed=seed)
    return w, synth.make_inputs(w)


@pytest.mark.parametrize("gate", ["softplus", "safe"])
def test_zero_state_one_token_closed_form(gate):
    """From a zero state, one token of the rule gives S_1 = beta k v^T (the decay acts on
    zero and the prediction u is zero) and o = S_1^T q = beta (k . q) v. With identity conv
    taps (tap 3 = 1, the rest 0) the activations are SiLU of the token itself, so q, k and v
    come from the input channels through library routines alone: q = scale * normalize(
    silu(x_q[h])), k = normalize(silu(x_k[h])), v = silu(x_v[hv]), h = hv // (HV / H). This
    fixes which channels play q, k and v, and the head map, against the page's formula."""
    w, inp = _small_inputs(N=2, T=1, H=2, HV=4, K=8, V=6, seed=3, gate=gate)
    C = w.C
    cw = torch.zeros(C, 4)
    cw[:, 3] = 1.0
    inp["conv_weight"] = cw
    inp["state"] = torch.zeros_like(inp["state"])
    scale = 0.3
    out = oracle.verify(inp, H=w.H, HV=w.HV, K=w.K, V=w.V,
                        gate_mode=oracle.GATE_SAFE if gate == "safe" else oracle.GATE_SOFTPLUS, scale=scale, eps=0.0)
    x = torch.as_tensor(oracle.f64(inp["mixed_qkv"]))
    act = F.silu(x)
    beta = torch.sigmoid(torch.as_tensor(oracle.f64(inp["beta"])))
    g = w.HV // w.H
    for n in range(w.N):
        for hv in range(w.HV):
            h = hv // g
            q = scale * F.normalize(act[n, 0, h * w.K:(h + 1) * w.K], dim=0)
            k = F.normalize(act[n, 0, (w.H + h) * w.K:(w.H + h + 1) * w.K], dim=0)
            v = act[n, 0, 2 * w.H * w.K + hv * w.V:2 * w.H * w.K + (hv + 1) * w.V]
            b = beta[n, 0, hv]
            np.testing.assert_allclose(out["inter_ssm"][n, 0, hv], (b * torch.outer(k, v)).numpy(), rtol=1e-12,
                                       atol=1e-15)
            np.testing.assert_allclose(out["o"][n, 0, hv], (b * torch.dot(k, q) * v).numpy(), rtol=1e-12,
                                       atol=1e-15)


@pytest.mark.parametrize("gate", ["softplus", "safe"])
def test_beta0_alpha1_leaves_state(gate):
    """beta = 0 (raw -inf) and no decay (raw gate -inf): every snapshot equals the state,
    and o_t = state^T q_t with q_t from the conv + normalisation alone."""
    w, inp = _small_inputs(gate=gate)
    inp["beta"] = torch.full_like(inp["beta"], -math.inf)
    inp["gate"] = torch.full_like(inp["gate"], -math.inf)
    out = oracle.verify_workload(w, inp)
    st = oracle.f64(inp["state"])
    for t in range(w.T):
        np.testing.assert_array_equal(out["inter_ssm"][:, t], st)
    act = oracle.conv_silu(inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"])
    for n in range(w.N):
        for t in range(w.T):
            for hv in range(w.HV):
                q = oracle.l2norm(act[n, t, hv * w.K:(hv + 1) * w.K], scale=w.K ** -0.5)
                np.testing.assert_allclose(out["o"][n, t, hv], st[n, hv].T @ q, atol=1e-14)


def test_beta0_gives_pure_decay():
    """beta = 0: S_t = Diag(prod_{tau <= t} alpha_tau) S_0."""
    w, inp = _small_inputs(T=4, gate="safe")
    inp["beta"] = torch.full_like(inp["beta"], -math.inf)
    out = oracle.verify_workload(w, inp)
    g = oracle.f64(inp["gate"])
    st = oracle.f64(inp["state"])
    A, dtb = oracle.f64(inp["A_log"]), oracle.f64(inp["dt_bias"])
    for n in range(w.N):
        for hv in range(w.HV):
            cum = np.ones(w.K)
            for t in range(w.T):
                cum = cum * np.exp([oracle.log_decay(1, g[n, t, hv, i], dtb[hv * w.K + i], A[hv]) for i in range(w.K)])
                np.testing.assert_allclose(out["inter_ssm"][n, t, hv], cum[:, None] * st[n, hv], rtol=1e-13, atol=1e-15)


def test_scale_only_scales_output():
    """The q scale multiplies o and leaves the state snapshots alone."""
    w, inp = _small_inputs()
    a = oracle.verify_workload(w, inp, scale=0.25)
    b = oracle.verify_workload(w, inp, scale=0.5)
    np.testing.assert_array_equal(a["inter_ssm"], b["inter_ssm"])
    np.testing.assert_allclose(b["o"], 2.0 * a["o"], rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("gate", ["softplus", "safe"])
@pytest.mark.parametrize("HV", [2, 4])
def test_chained_single_token_calls(gate, HV):
    """A T-token verify equals T chained one-token calls that feed back the snapshot and
    the rolled conv cache (the repeated verify chains of PR#107 Tests & Accuracy)."""
    T = 4
    w, inp = _small_inputs(T=T, HV=HV, gate=gate, seed=11)
    full = oracle.verify_workload(w, inp)
    w1 = w.with_(T=1)
    cs, st = inp["conv_state"], inp["state"]
    for t in range(T):
        step = {k: v for k, v in inp.items()}
        step["mixed_qkv"] = inp["mixed_qkv"][:, t:t + 1]
        step["gate"] = inp["gate"][:, t:t + 1]
        step["beta"] = inp["beta"][:, t:t + 1]
        step["conv_state"], step["state"] = cs, st
        out = oracle.verify_workload(w1, step)
        np.testing.assert_allclose(out["inter_ssm"][:, 0], full["inter_ssm"][:, t], rtol=0, atol=1e-13)
        np.testing.assert_allclose(out["o"][:, 0], full["o"][:, t], rtol=0, atol=1e-13)
        np.testing.assert_array_equal(out["conv_window"][:, 0], full["conv_window"][:, t])
        cs, st = torch.from_numpy(out["conv_state"]), torch.from_numpy(out["inter_ssm"][:, 0])
    np.testing.assert_array_equal(cs.numpy(), full["conv_state"])


def _expand_gva(w, inp):
    """The same problem with every value head given its own copy of its q/k head
    (repeat-interleave: value head hv reads q/k head hv // g)."""
    H, HV, K, g = w.H, w.HV, w.K, w.HV // w.H
    qk_idx = []
    for blk in range(2):  # q block, k block
        for hv in range(HV):
            h = hv // g
            qk_idx.extend(range(blk * H * K + h * K, blk * H * K + (h + 1) * K))
    idx = torch.tensor(qk_idx + list(range(2 * H * K, w.C)))
    e = dict(inp)
    e["mixed_qkv"] = inp["mixed_qkv"][:, :, idx]
    e["conv_weight"] = inp["conv_weight"][idx]
    e["conv_state"] = inp["conv_state"][:, idx]
    return w.with_(H=HV), e, idx


@pytest.mark.parametrize("H,HV", [(1, 2), (2, 4), (1, 4)])
def test_gva_equals_head_repetition(H, HV):
    w, inp = _small_inputs(H=H, HV=HV, T=3, seed=21)
    out = oracle.verify_workload(w, inp)
    we, ie, idx = _expand_gva(w, inp)
    oute = oracle.verify_workload(we, ie)
    np.testing.assert_array_equal(out["o"], oute["o"])
    np.testing.assert_array_equal(out["inter_ssm"], oute["inter_ssm"])
    np.testing.assert_array_equal(out["conv_window"][:, :, idx.numpy()], oute["conv_window"])
    np.testing.assert_array_equal(out["conv_state"][:, idx.numpy()], oute["conv_state"])


def _torch_reference(w, inp):
    """An independent float64 statement of the step from torch library pieces:
    depthwise conv1d, silu, softplus(beta, threshold), sigmoid and dense matrix products."""
    d = torch.float64
    x = inp["mixed_qkv"].to(d)
    N, T, C = x.shape
    H, HV, K, V, g = w.H, w.HV, w.K, w.V, w.HV // w.H
    E = torch.cat([inp["conv_state"].to(d), x.transpose(1, 2)], dim=2)  # [N, C, T+3]
    act = F.silu(F.conv1d(E, inp["conv_weight"].to(d).unsqueeze(1), groups=C)).transpose(1, 2)  # [N,T,C]
    q = act[..., :H * K].reshape(N, T, H, K)
    k = act[..., H * K:2 * H * K].reshape(N, T, H, K)
    v = act[..., 2 * H * K:].reshape(N, T, HV, V)
    q = q * torch.rsqrt((q * q).sum(-1, keepdim=True) + synth.L2NORM_EPS) * K ** -0.5
    k = k * torch.rsqrt((k * k).sum(-1, keepdim=True) + synth.L2NORM_EPS)
    q = q.repeat_interleave(g, dim=2)
    k = k.repeat_interleave(g, dim=2)
    gam = inp["gate"].to(d) + inp["dt_bias"].to(d).reshape(HV, K)
    eA = torch.exp(inp["A_log"].to(d)).reshape(1, 1, HV, 1)
    if w.gate == "softplus":
        ld = -eA * F.softplus(gam, beta=synth.SOFTPLUS_BETA, threshold=synth.SOFTPLUS_THRESHOLD)
    else:
        ld = synth.LOWER_BOUND * torch.sigmoid(eA * gam)
    alpha = torch.exp(ld)
    beta = torch.sigmoid(inp["beta"].to(d))
    S = inp["state"].to(d).clone()
    I = torch.eye(K, dtype=d)
    o = torch.empty(N, T, HV, V, dtype=d)
    snaps = torch.empty(N, T, HV, K, V, dtype=d)
    for t in range(T):
        kt = k[:, t].unsqueeze(-1)  # [N,HV,K,1]
        b = beta[:, t].reshape(N, HV, 1, 1)
        A = (I - b * (kt @ kt.transpose(-1, -2))) @ torch.diag_embed(alpha[:, t])
        S = A @ S + b * (kt @ v[:, t].unsqueeze(-2))
        snaps[:, t] = S
        o[:, t] = (S.transpose(-1, -2) @ q[:, t].unsqueeze(-1)).squeeze(-1)
    return o.numpy(), snaps.numpy()


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("gva_small", dict(N=3, T=5, H=2, HV=4, K=16, V=8, gate="safe")),
    ("t1", dict(N=2, T=1, H=1, HV=3, K=8, V=12)),
])
def test_matches_independent_torch_composition(name, kw):
    if name == "tiny":
        w = synth.WORKLOADS["tiny"]
        inp = synth.make_inputs(w)
    else:
        w, inp = _small_inputs(seed=31, **kw)
    out = oracle.verify_workload(w, inp)
    o, snaps = _torch_reference(w, inp)
    np.testing.assert_allclose(out["o"], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["inter_ssm"], snaps, rtol=1e-12, atol=1e-13)


def test_no_nan_at_extreme_gate_and_beta():
    w, inp = _small_inputs(T=3)
    for gate in ("softplus", "safe"):
        ww = w.with_(gate=gate)
        inp["gate"] = torch.tensor([1e4, -1e4, 3e38]).repeat(inp["gate"].numel() // 3 + 1)[: inp["gate"].numel()].reshape(inp["gate"].shape)
        inp["beta"] = torch.full_like(inp["beta"], 1e4)
        out = oracle.verify_workload(ww, inp)
        assert np.all(np.isfinite(out["o"])) and np.all(np.isfinite(out["inter_ssm"]))


def test_zero_q_k_head_is_finite():
    w, inp = _small_inputs()
    inp["conv_weight"][: 2 * w.H * w.K] = 0.0  # q and k channels convolve to 0
    out = oracle.verify_workload(w, inp)
    assert np.all(np.isfinite(out["o"]))
    # k = 0 -> no write, q = 0 -> o = 0: snapshots are pure decay, outputs vanish
    assert np.all(out["o"] == 0.0)


def test_rejects_bad_shapes():
    w, inp = _small_inputs(H=2, HV=3)  # HV must be a multiple of H
    with pytest.raises(ValueError):
        oracle.verify_workload(w, inp)


def test_tiny_regression_fixture():
    """tests/golden/tiny_oracle.json was written by tests/golden/make_golden.py from this
    oracle; it catches any later change to the oracle's arithmetic."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")) as f:
        doc = json.load(f)
    w = synth.WORKLOADS["tiny"]
    out = oracle.verify_workload(w, synth.make_inputs(w))
    np.testing.assert_allclose(out["o"].reshape(-1), doc["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["inter_ssm"].sum(axis=(2, 3, 4)).reshape(-1), doc["inter_ssm_sum_by_nt"], rtol=1e-12)
    np.testing.assert_allclose(out["inter_ssm"][:, :, :, 0, :].reshape(-1), doc["inter_ssm_first_row"], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(out["conv_state"].reshape(-1), doc["conv_state"])


# ---------------------------------------------------------------- pooled verify and commit
def _pool_case(seed=41, N=4, T=3, H=2, HV=4, K=8, V=8, slots=(7, 6, 9), gate="safe"):
    w, inp = _small_inputs(N=N, T=T, H=H, HV=HV, K=K, V=V, seed=seed, gate=gate)
    r = np.random.default_rng(seed)
    Pc, Ps, Pi = slots
    cs_idx = r.permutation(Pc)[:N]
    st_idx = r.permutation(Ps)[:N]
    in_idx = r.permutation(Pi)[:N]
    cs_pool = r.normal(size=(Pc, w.C, 3))
    st_pool = r.normal(size=(Ps, HV, K, V)) * 0.1
    cs_pool[cs_idx] = oracle.f64(inp["conv_state"])
    st_pool[st_idx] = oracle.f64(inp["state"])
    pools = {
        "conv_state_indices": cs_idx, "cache_indices": st_idx, "intermediate_state_indices": in_idx,
        "o": r.normal(size=(N, T, HV, V)), "inter_ssm": r.normal(size=(Pi, T, HV, K, V)),
        "conv_window": r.normal(size=(Pi, T, w.C, 3)),
    }
    pinp = dict(inp)
    pinp["conv_state"], pinp["state"] = cs_pool, st_pool
    return w, inp, pinp, pools


def _gm(w):
    return oracle.GATE_SAFE if w.gate == "safe" else oracle.GATE_SOFTPLUS


def test_pooled_identity_equals_dense():
    w, inp = _small_inputs(N=3, T=4, H=1, HV=2)
    dense = oracle.verify_workload(w, inp)
    pools = {"o": np.zeros((w.N, w.T, w.HV, w.V)), "inter_ssm": np.zeros((w.N, w.T, w.HV, w.K, w.V)),
             "conv_window": np.zeros((w.N, w.T, w.C, 3))}
    got = oracle.verify_pooled(inp, pools, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    for k in dense:
        np.testing.assert_array_equal(got[k], dense[k])


def test_pooled_rows_scatter_and_untouched_rows_keep():
    """Per-sequence results land in the rows the index arrays name; other rows keep their contents."""
    w, inp, pinp, pools = _pool_case()
    dense = oracle.verify_workload(w, inp)
    got = oracle.verify_pooled(pinp, pools, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    cs_i, in_i = pools["conv_state_indices"], pools["intermediate_state_indices"]
    np.testing.assert_array_equal(got["o"], dense["o"])
    np.testing.assert_array_equal(got["inter_ssm"][in_i], dense["inter_ssm"])
    np.testing.assert_array_equal(got["conv_window"][in_i], dense["conv_window"])
    np.testing.assert_array_equal(got["conv_state"][cs_i], dense["conv_state"])
    other_i = np.setdiff1d(np.arange(pools["inter_ssm"].shape[0]), in_i)
    np.testing.assert_array_equal(got["inter_ssm"][other_i], pools["inter_ssm"][other_i])
    other_c = np.setdiff1d(np.arange(pinp["conv_state"].shape[0]), cs_i)
    np.testing.assert_array_equal(got["conv_state"][other_c], pinp["conv_state"][other_c])


def test_pooled_padding_entries_are_skipped():
    w, inp, pinp, pools = _pool_case(seed=43)
    pools["cache_indices"] = pools["cache_indices"].copy()
    pools["cache_indices"][1] = -1
    pools["intermediate_state_indices"] = pools["intermediate_state_indices"].copy()
    pools["intermediate_state_indices"][2] = pools["inter_ssm"].shape[0]  # one past the end
    got = oracle.verify_pooled(pinp, pools, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    for n in (1, 2):
        np.testing.assert_array_equal(got["o"][n], pools["o"][n])
        c = pools["conv_state_indices"][n]
        np.testing.assert_array_equal(got["conv_state"][c], pinp["conv_state"][c])
    np.testing.assert_array_equal(got["inter_ssm"][pools["intermediate_state_indices"][1]],
                                  pools["inter_ssm"][pools["intermediate_state_indices"][1]])


@pytest.mark.parametrize("a", [1, 2, 3])
def test_commit_equals_verify_of_the_accepted_prefix(a):
    """Accepting a of T tokens leaves the state and conv cache a dense verify of just those
    a tokens produces (an independent run of the step on the shorter input)."""
    w, inp, pinp, pools = _pool_case(seed=47)
    got = oracle.verify_pooled(pinp, pools, H=w.H, HV=w.HV, K=w.K, V=w.V, gate_mode=_gm(w))
    acc = np.full(w.N, a)
    acc[0] = 0  # nothing accepted: left alone
    c = oracle.commit(acc, pools, got["inter_ssm"], got["conv_window"], pinp["state"], got["conv_state"], T=w.T)
    wa = w.with_(T=a)
    pre = dict(inp)
    pre["mixed_qkv"], pre["gate"], pre["beta"] = inp["mixed_qkv"][:, :a], inp["gate"][:, :a], inp["beta"][:, :a]
    ref = oracle.verify_workload(wa, pre)
    cs_i, st_i = pools["conv_state_indices"], pools["cache_indices"]
    for n in range(1, w.N):
        np.testing.assert_array_equal(c["state"][st_i[n]], ref["inter_ssm"][n, a - 1])
        np.testing.assert_array_equal(c["conv_state"][cs_i[n]], ref["conv_state"][n])
    np.testing.assert_array_equal(c["state"][st_i[0]], pinp["state"][st_i[0]])
    np.testing.assert_array_equal(c["conv_state"][cs_i[0]], got["conv_state"][cs_i[0]])
