"""Python face of the float64 CPU oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use this module to say what the fused conv1d + KDA verify step must
return. The product path (the HIP library and its binding) never imports it.

The C source is compiled with gcc into ``libkda_oracle.so`` next to this file
(``build()``); ``load()`` builds it only if it is missing. Inputs may be numpy
arrays or CPU torch tensors of any float dtype; they are upcast exactly to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib: Optional[ctypes.CDLL] = None

GATE_SOFTPLUS = 0
GATE_SAFE = 1

_D = ctypes.c_double
_I = ctypes.c_int
_P = ctypes.POINTER(ctypes.c_double)


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_silu.argtypes = [_D]
    lib.oracle_silu.restype = _D
    lib.oracle_sigmoid.argtypes = [_D]
    lib.oracle_sigmoid.restype = _D
    lib.oracle_softplus.argtypes = [_D, _D, _D]
    lib.oracle_softplus.restype = _D
    lib.oracle_log_decay.argtypes = [_I, _D, _D, _D, _D, _D, _D]
    lib.oracle_log_decay.restype = _D
    lib.oracle_l2norm.argtypes = [_I, _P, _D, _D, _P]
    lib.oracle_l2norm.restype = None
    lib.oracle_conv_silu.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    lib.oracle_conv_silu.restype = None
    lib.oracle_conv_roll.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    lib.oracle_conv_roll.restype = None
    lib.oracle_delta_step.argtypes = [_I, _I, _P, _P, _P, _P, _D, _P, _P]
    lib.oracle_delta_step.restype = None
    lib.oracle_verify.argtypes = [_I] * 7 + [_D] * 5 + [_P] * 12
    lib.oracle_verify.restype = _I
    _lib = lib
    return lib


def f64(x) -> np.ndarray:
    """Exact upcast to a C-contiguous float64 numpy array."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_P)


# ----------------------------------------------------------------------------------
# Scalar and per-step entry points (each is one step of the method, see kda_oracle.c)
# ----------------------------------------------------------------------------------
def silu(y: float) -> float:
    return load().oracle_silu(float(y))


def sigmoid(x: float) -> float:
    return load().oracle_sigmoid(float(x))


def softplus(x: float, beta: float = 1.0, threshold: float = 20.0) -> float:
    return load().oracle_softplus(float(x), float(beta), float(threshold))


def log_decay(mode: int, g: float, dt_bias: float, A_log: float, lower_bound: float = -5.0,
              softplus_beta: float = 1.0, softplus_threshold: float = 20.0) -> float:
    return load().oracle_log_decay(int(mode), float(g), float(dt_bias), float(A_log),
                                   float(lower_bound), float(softplus_beta), float(softplus_threshold))


def l2norm(x, eps: float = 1e-6, scale: float = 1.0) -> np.ndarray:
    x = f64(x).reshape(-1)
    out = np.empty_like(x)
    load().oracle_l2norm(x.size, _ptr(x), float(eps), float(scale), _ptr(out))
    return out


def conv_silu(mixed_qkv, conv_weight, conv_state) -> np.ndarray:
    """act[N,T,C] = SiLU(width-4 causal conv over (conv_state, mixed_qkv))."""
    x, w, s = f64(mixed_qkv), f64(conv_weight), f64(conv_state)
    N, T, C = x.shape
    assert w.shape == (C, 4) and s.shape == (N, C, 3)
    act = np.empty((N, T, C))
    load().oracle_conv_silu(N, T, C, _ptr(x), _ptr(w), _ptr(s), _ptr(act))
    return act


def conv_roll(mixed_qkv, conv_state):
    """(conv_window[N,T,C,3], conv_state_out[N,C,3]): raw-value copies, no arithmetic."""
    x, s = f64(mixed_qkv), f64(conv_state)
    N, T, C = x.shape
    assert s.shape == (N, C, 3)
    cw = np.empty((N, T, C, 3))
    cs = np.empty((N, C, 3))
    load().oracle_conv_roll(N, T, C, _ptr(x), _ptr(s), _ptr(cw), _ptr(cs))
    return cw, cs


def delta_step(S, alpha, k, v, beta: float, q):
    """One token of the gated delta rule. Returns (S_new[K,V], o[V]); S is not modified."""
    S = f64(S).copy()
    K, V = S.shape
    a, kk, vv, qq = f64(alpha), f64(k), f64(v), f64(q)
    assert a.shape == (K,) and kk.shape == (K,) and vv.shape == (V,) and qq.shape == (K,)
    o = np.empty(V)
    load().oracle_delta_step(K, V, _ptr(S), _ptr(a), _ptr(kk), _ptr(vv), float(beta), _ptr(qq), _ptr(o))
    return S, o


def verify(inputs: Dict, *, H: int, HV: int, K: int, V: int, gate_mode: int,
           lower_bound: float = -5.0, softplus_beta: float = 1.0, softplus_threshold: float = 20.0,
           scale: Optional[float] = None, eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """The whole verify step on float64 copies of ``inputs``.

    ``inputs`` holds mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state
    (the keys of ``synth.make_inputs``). Returns float64 arrays o, inter_ssm,
    conv_window and conv_state (the rolled cache; the input is not modified).
    """
    x = f64(inputs["mixed_qkv"])
    N, T, C = x.shape
    assert C == 2 * H * K + HV * V, "mixed_qkv width must be 2*H*K + HV*V"
    arrs = [x] + [f64(inputs[k]) for k in ("conv_weight", "conv_state", "gate", "A_log",
                                            "dt_bias", "beta", "state")]
    assert arrs[1].shape == (C, 4) and arrs[2].shape == (N, C, 3)
    assert arrs[3].shape == (N, T, HV, K) and arrs[4].shape == (HV,)
    assert arrs[5].shape == (HV * K,) and arrs[6].shape == (N, T, HV)
    assert arrs[7].shape == (N, HV, K, V)
    if scale is None:
        scale = K ** -0.5
    out = {
        "o": np.empty((N, T, HV, V)),
        "inter_ssm": np.empty((N, T, HV, K, V)),
        "conv_window": np.empty((N, T, C, 3)),
        "conv_state": np.empty((N, C, 3)),
    }
    rc = load().oracle_verify(N, T, H, HV, K, V, int(gate_mode), float(lower_bound),
                              float(softplus_beta), float(softplus_threshold), float(scale), float(eps),
                              *[_ptr(a) for a in arrs], _ptr(out["o"]), _ptr(out["inter_ssm"]),
                              _ptr(out["conv_window"]), _ptr(out["conv_state"]))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected the shape (rc={rc})")
    return out


def verify_workload(w, inputs: Dict, **kw) -> Dict[str, np.ndarray]:
    """``verify`` with the shape and gate form taken from a ``synth.Workload``."""
    return verify(inputs, H=w.H, HV=w.HV, K=w.K, V=w.V,
                  gate_mode=GATE_SAFE if w.gate == "safe" else GATE_SOFTPLUS, **kw)


def verify_pooled(inputs: Dict, pools: Dict, *, H: int, HV: int, K: int, V: int, gate_mode: int,
                  **kw) -> Dict[str, np.ndarray]:
    """The verify step on pooled buffers (PR#107 PR description: conv_state_indices,
    cache_indices and intermediate_state_indices, each normalised on its own).

    ``inputs`` holds the per-call tensors (mixed_qkv, conv_weight, gate, A_log, dt_bias,
    beta) and the pools ``conv_state`` [Pc,C,3] and ``state`` [Ps,HV,K,V]; ``pools`` holds
    the index arrays (None = identity) and the initial contents of the written pools
    ``inter_ssm`` [Pi,T,HV,K,V], ``conv_window`` [Pi,T,C,3] and of ``o`` [N,T,HV,V].
    Sequence n is padding (skipped) when any of its indices is outside its pool. Each
    sequence is gathered, run through ``verify`` and scattered back. Returns float64
    copies of o, inter_ssm, conv_window and conv_state after the call.
    """
    x = f64(inputs["mixed_qkv"])
    N = x.shape[0]
    cs_pool = f64(inputs["conv_state"]).copy()
    st_pool = f64(inputs["state"])
    out_o = f64(pools["o"]).copy()
    out_is = f64(pools["inter_ssm"]).copy()
    out_cw = f64(pools["conv_window"]).copy()

    def rows(key, slots):
        idx = pools.get(key)
        return np.arange(N) if idx is None else np.asarray(f64(idx), dtype=np.int64)

    cs_i = rows("conv_state_indices", cs_pool.shape[0])
    st_i = rows("cache_indices", st_pool.shape[0])
    in_i = rows("intermediate_state_indices", out_is.shape[0])
    for n in range(N):
        c, s_, i = cs_i[n], st_i[n], in_i[n]
        if not (0 <= c < cs_pool.shape[0] and 0 <= s_ < st_pool.shape[0] and 0 <= i < out_is.shape[0]):
            continue
        one = {
            "mixed_qkv": x[n:n + 1], "conv_weight": inputs["conv_weight"],
            "conv_state": cs_pool[c:c + 1], "gate": f64(inputs["gate"])[n:n + 1],
            "A_log": inputs["A_log"], "dt_bias": inputs["dt_bias"],
            "beta": f64(inputs["beta"])[n:n + 1], "state": st_pool[s_:s_ + 1],
        }
        r = verify(one, H=H, HV=HV, K=K, V=V, gate_mode=gate_mode, **kw)
        out_o[n] = r["o"][0]
        out_is[i] = r["inter_ssm"][0]
        out_cw[i] = r["conv_window"][0]
        cs_pool[c] = r["conv_state"][0]
    return {"o": out_o, "inter_ssm": out_is, "conv_window": out_cw, "conv_state": cs_pool}


def commit(accepted, pools: Dict, inter_ssm, conv_window, state, conv_state, T: int) -> Dict[str, np.ndarray]:
    """Accept step: for each sequence n with 1 <= a_n <= T (and valid indices),
    state[cache_indices[n]] <- inter_ssm[intermediate_state_indices[n], a_n - 1] and
    conv_state[conv_state_indices[n]] <- conv_window[intermediate_state_indices[n], a_n - 1].
    Returns float64 copies of the state and conv_state pools."""
    acc = np.asarray(f64(accepted), dtype=np.int64)
    N = acc.shape[0]
    isp, cwp = f64(inter_ssm), f64(conv_window)
    st, cs = f64(state).copy(), f64(conv_state).copy()

    def rows(key):
        idx = pools.get(key) if pools else None
        return np.arange(N) if idx is None else np.asarray(f64(idx), dtype=np.int64)

    cs_i, st_i, in_i = rows("conv_state_indices"), rows("cache_indices"), rows("intermediate_state_indices")
    for n in range(N):
        a, c, s_, i = acc[n], cs_i[n], st_i[n], in_i[n]
        if not (1 <= a <= T and 0 <= c < cs.shape[0] and 0 <= s_ < st.shape[0] and 0 <= i < isp.shape[0]):
            continue
        st[s_] = isp[i, a - 1]
        cs[c] = cwp[i, a - 1]
    return {"state": st, "conv_state": cs}
