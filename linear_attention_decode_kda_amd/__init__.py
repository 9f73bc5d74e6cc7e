"""MI355X (gfx950) fused causal-conv1d + KDA multi-token verify-decode step.

A thin ctypes binding over ``libkda_verify.so`` (C ABI in include/kda_verify.h).
Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their pointers and the current HIP stream are handed to the
library, which does every step of the computation in its kernels. There is no
fallback: if the library is missing or fails to load, every call raises.

Operation: cuLA pull request page "[KDA] Fuse causal conv1d into MTP verify decode
#107" (PR description).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch  # loads the HIP runtime the library binds to

from . import synth  # noqa: F401  (seeded inputs; no arithmetic of the step)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda_verify.so")

KDA_OK = 0
STATUS = {
    0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_UNSUPPORTED",
    -4: "KDA_ERR_ALIGN", -5: "KDA_ERR_WORKSPACE", -6: "KDA_ERR_LAUNCH", -7: "KDA_ERR_ALIAS",
    -8: "KDA_ERR_SCRATCH",
}
F32, BF16 = 0, 1
GATE_SOFTPLUS, GATE_SAFE = 0, 1
VARIANT_AUTO, VARIANT_SMALL, VARIANT_LARGE = 0, 1, 2
MAX_T = 16
NOALLOC_SCRATCH_BYTES = 262144  # KDA_NOALLOC_SCRATCH_BYTES


class Params(ctypes.Structure):
    """Mirror of ``kda_verify_params``."""

    _fields_ = [
        ("N", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("gate_mode", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("lower_bound", ctypes.c_float), ("softplus_beta", ctypes.c_float),
        ("softplus_threshold", ctypes.c_float), ("scale", ctypes.c_float), ("l2norm_eps", ctypes.c_float),
        ("tile_columns", ctypes.c_int32), ("store_policy", ctypes.c_int32),
        ("max_wg_per_cu", ctypes.c_int32), ("column_groups", ctypes.c_int32), ("schedule", ctypes.c_int32),
        ("unit_order", ctypes.c_int32), ("prefetch", ctypes.c_int32),
    ]


class PoolDesc(ctypes.Structure):
    """Mirror of ``kda_pool_desc``."""

    _fields_ = [
        ("conv_state_indices", ctypes.c_void_p), ("cache_indices", ctypes.c_void_p),
        ("intermediate_state_indices", ctypes.c_void_p), ("conv_state_slots", ctypes.c_int32),
        ("state_slots", ctypes.c_int32), ("intermediate_slots", ctypes.c_int32),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({lib_status_string(status)})")


_lib: Optional[ctypes.CDLL] = None
_VP = ctypes.c_void_p
_SZ = ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m linear_attention_decode_kda_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    PP = ctypes.POINTER(Params)
    lib.kda_verify_params_init.argtypes = [PP] + [ctypes.c_int32] * 6
    lib.kda_verify_params_init.restype = None
    lib.kda_workspace_bytes.argtypes = [PP]
    lib.kda_workspace_bytes.restype = _SZ
    lib.kda_workspace_reset.argtypes = [_VP, _SZ, _VP]
    lib.kda_workspace_reset.restype = ctypes.c_int
    lib.kda_select_variant.argtypes = [PP]
    lib.kda_select_variant.restype = ctypes.c_int32
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.kda_select_launch.argtypes = [PP, I32P, I32P, I32P, I32P, I32P, I32P, I32P]
    lib.kda_select_launch.restype = ctypes.c_int
    lib.kda_validate.argtypes = [PP] + [_VP] * 12 + [_SZ]
    lib.kda_validate.restype = ctypes.c_int
    lib.kda_conv_verify_decode.argtypes = [PP] + [_VP] * 12 + [_SZ, _VP]
    lib.kda_conv_verify_decode.restype = ctypes.c_int
    PD = ctypes.POINTER(PoolDesc)
    lib.kda_conv_verify_decode_pooled.argtypes = [PP, PD] + [_VP] * 12 + [_SZ, _VP]
    lib.kda_conv_verify_decode_pooled.restype = ctypes.c_int
    lib.kda_conv_verify_decode_unfused.argtypes = [PP, PD] + [_VP] * 13 + [_SZ, _VP]
    lib.kda_conv_verify_decode_unfused.restype = ctypes.c_int
    lib.kda_conv_verify_decode_noalloc.argtypes = [PP] + [_VP] * 11 + [_VP]
    lib.kda_conv_verify_decode_noalloc.restype = ctypes.c_int
    lib.kda_verify_commit.argtypes = [PP, PD] + [_VP] * 5 + [_VP]
    lib.kda_verify_commit.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int32]
    lib.kda_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def lib_status_string(status: int) -> str:
    try:
        return load().kda_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def make_params(N: int, T: int, H: int, HV: int, K: int, V: int, *, dtype: str = "bf16",
                gate: str = "softplus", variant: int = VARIANT_AUTO, lower_bound: float = -5.0,
                softplus_beta: float = 1.0, softplus_threshold: float = 20.0, scale: float = 0.0,
                l2norm_eps: float = 1e-6, tile_columns: int = 0, store_policy: int = 0,
                max_wg_per_cu: int = 0, column_groups: int = 0, schedule: int = 0, unit_order: int = 0,
                prefetch: int = 0) -> Params:
    p = Params()
    load().kda_verify_params_init(ctypes.byref(p), N, T, H, HV, K, V)
    p.in_dtype = {"f32": F32, "bf16": BF16}[dtype]
    p.gate_mode = {"softplus": GATE_SOFTPLUS, "safe": GATE_SAFE}[gate]
    p.variant = int(variant)
    p.lower_bound = lower_bound
    p.softplus_beta = softplus_beta
    p.softplus_threshold = softplus_threshold
    p.scale = scale
    p.l2norm_eps = l2norm_eps
    p.tile_columns = tile_columns
    p.store_policy = store_policy
    p.max_wg_per_cu = max_wg_per_cu
    p.column_groups = column_groups
    p.schedule = schedule
    p.unit_order = unit_order
    p.prefetch = prefetch
    return p


def params_for(w, **kw) -> Params:
    """Params of a ``synth.Workload``."""
    return make_params(w.N, w.T, w.H, w.HV, w.K, w.V, dtype=w.dtype, gate=w.gate, **kw)


def workspace_bytes(p: Params) -> int:
    return int(load().kda_workspace_bytes(ctypes.byref(p)))


def select_variant(p: Params) -> int:
    return int(load().kda_select_variant(ctypes.byref(p)))


def select_launch(p: Params) -> Dict[str, int]:
    """The launch configuration the library picks for ``p``: tile_columns, store_policy
    (1 streaming, 2 streaming at device scope), max_wg_per_cu (0 = no cap), column_groups, schedule
    (1 grid, 2 queue, 3 stream), unit_order (1 XCD ranges, 2 pairs) and prefetch (the stream's
    state load: 1 after the conv, 2 at the start; 0 for the other schedules)."""
    t, s, o, g, q, u, f = (ctypes.c_int32() for _ in range(7))
    st = load().kda_select_launch(ctypes.byref(p), ctypes.byref(t), ctypes.byref(s), ctypes.byref(o),
                                  ctypes.byref(g), ctypes.byref(q), ctypes.byref(u), ctypes.byref(f))
    if st != KDA_OK:
        raise KdaError(st, "kda_select_launch")
    return {"tile_columns": t.value, "store_policy": s.value, "max_wg_per_cu": o.value,
            "column_groups": g.value, "schedule": q.value, "unit_order": u.value, "prefetch": f.value}


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def workspace_reset(ws: torch.Tensor, stream=None) -> None:
    st = load().kda_workspace_reset(_VP(ws.data_ptr()), ws.numel() * ws.element_size(), _VP(_stream(stream)))
    if st != KDA_OK:
        raise KdaError(st, "kda_workspace_reset")


def alloc_workspace(p: Params, device="cuda") -> torch.Tensor:
    """A zeroed workspace for ``p`` (uint8 tensor; the counters zero themselves after each call)."""
    ws = torch.empty(max(workspace_bytes(p), 256), dtype=torch.uint8, device=device)
    workspace_reset(ws)
    return ws


_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}


def _check(name, t: torch.Tensor, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _verify_args(p: Params, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                 o, inter_ssm, conv_window, workspace):
    """Check the tensors of a verify call against ``p``; returns their 12 device pointers."""
    N, T, H, HV, K, V = p.N, p.T, p.H, p.HV, p.K, p.V
    C = 2 * H * K + HV * V
    dt = _TORCH_DT.get(p.in_dtype)
    if dt is None:
        raise KdaError(-3, "kda_conv_verify_decode")
    _check("mixed_qkv", mixed_qkv, (N, T, C), dt)
    _check("conv_weight", conv_weight, (C, 4), dt)
    _check("conv_state", conv_state, (N, C, 3), dt)
    _check("gate", gate, (N, T, HV, K), dt)
    _check("A_log", A_log, (HV,), torch.float32)
    _check("dt_bias", dt_bias, (HV * K,), torch.float32)
    _check("beta", beta, (N, T, HV), dt)
    _check("state", state, (N, HV, K, V), torch.float32)
    _check("o", o, (N, T, HV, V), dt)
    _check("inter_ssm", inter_ssm, (N, T, HV, K, V), torch.float32)
    _check("conv_window", conv_window, (N, T, C, 3), dt)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    return [t.data_ptr() for t in (mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                                   o, inter_ssm, conv_window, workspace)]


def kda_conv_verify_decode(p: Params, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                           o, inter_ssm, conv_window, workspace, stream=None) -> None:
    """One fused verify step on the current (or given) stream; see include/kda_verify.h.

    Writes o, inter_ssm, conv_window, and conv_state in place. Raises KdaError on a
    non-OK status (nothing was launched in that case).
    """
    ptrs = _verify_args(p, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                        o, inter_ssm, conv_window, workspace)
    st = load().kda_conv_verify_decode(ctypes.byref(p), *ptrs, workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    if st != KDA_OK:
        raise KdaError(st, "kda_conv_verify_decode")


def kda_conv_verify_decode_noalloc(p: Params, mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta,
                                   state, o, inter_ssm, conv_window, stream=None) -> None:
    """``kda_conv_verify_decode`` without a workspace: the library keeps the counters in a
    static per-GPU array (see include/kda_verify.h). Calls that overlap on one GPU race."""
    N, T, H, HV, K, V = p.N, p.T, p.H, p.HV, p.K, p.V
    C = 2 * H * K + HV * V
    dt = _TORCH_DT.get(p.in_dtype)
    if dt is None:
        raise KdaError(-3, "kda_conv_verify_decode_noalloc")
    for name, t, shape, tdt in (("mixed_qkv", mixed_qkv, (N, T, C), dt), ("conv_weight", conv_weight, (C, 4), dt),
                                ("conv_state", conv_state, (N, C, 3), dt), ("gate", gate, (N, T, HV, K), dt),
                                ("A_log", A_log, (HV,), torch.float32), ("dt_bias", dt_bias, (HV * K,), torch.float32),
                                ("beta", beta, (N, T, HV), dt), ("state", state, (N, HV, K, V), torch.float32),
                                ("o", o, (N, T, HV, V), dt), ("inter_ssm", inter_ssm, (N, T, HV, K, V), torch.float32),
                                ("conv_window", conv_window, (N, T, C, 3), dt)):
        _check(name, t, shape, tdt)
    ptrs = [t.data_ptr() for t in (mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state, o,
                                   inter_ssm, conv_window)]
    st = load().kda_conv_verify_decode_noalloc(ctypes.byref(p), *[_VP(x) for x in ptrs], _VP(_stream(stream)))
    if st != KDA_OK:
        raise KdaError(st, "kda_conv_verify_decode_noalloc")


class PreparedVerify:
    """``kda_conv_verify_decode`` bound to fixed tensors and a stream, for loops that reuse
    their buffers (a serving step, a benchmark): the argument checks run once, here, and
    each call is a single C call with the cached pointers. The caller keeps the tensors'
    storage in place while the object is used (it holds references, so they stay alive)."""

    def __init__(self, p: Params, inp: Dict[str, torch.Tensor], out: Dict[str, torch.Tensor],
                 workspace: torch.Tensor, stream=None):
        tensors = (inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"], inp["gate"], inp["A_log"],
                   inp["dt_bias"], inp["beta"], inp["state"], out["o"], out["inter_ssm"], out["conv_window"],
                   workspace)
        ptrs = _verify_args(p, *tensors)
        self.params = Params.from_buffer_copy(p)
        self._keep = tensors
        self._fn = load().kda_conv_verify_decode
        self._args = (ctypes.byref(self.params), *ptrs, workspace.numel() * workspace.element_size(),
                      _stream(stream))

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != KDA_OK:
            raise KdaError(st, "kda_conv_verify_decode")


def _index(name, t, N):
    if t is None:
        return None
    _check(name, t, (N,), torch.int32)
    return t


def make_pools(N: int, conv_state_indices=None, cache_indices=None, intermediate_state_indices=None,
               conv_state_slots=None, state_slots=None, intermediate_slots=None) -> PoolDesc:
    """A pool descriptor; each index array is an int32 [N] GPU tensor or None (identity)."""
    for name, t in (("conv_state_indices", conv_state_indices), ("cache_indices", cache_indices),
                    ("intermediate_state_indices", intermediate_state_indices)):
        _index(name, t, N)
    d = PoolDesc()
    d.conv_state_indices = conv_state_indices.data_ptr() if conv_state_indices is not None else None
    d.cache_indices = cache_indices.data_ptr() if cache_indices is not None else None
    d.intermediate_state_indices = (intermediate_state_indices.data_ptr()
                                    if intermediate_state_indices is not None else None)
    d.conv_state_slots = N if conv_state_slots is None else conv_state_slots
    d.state_slots = N if state_slots is None else state_slots
    d.intermediate_slots = N if intermediate_slots is None else intermediate_slots
    # the descriptor holds the index tensors it points into, so that they live as long as it
    # does (a temporary such as idx.cuda() would otherwise be freed, and its memory reused,
    # before the call that reads it)
    d.index_tensors = (conv_state_indices, cache_indices, intermediate_state_indices)
    return d


def kda_conv_verify_decode_pooled(p: Params, pools: PoolDesc, mixed_qkv, conv_weight, conv_state, gate, A_log,
                                  dt_bias, beta, state, o, inter_ssm, conv_window, workspace, stream=None) -> None:
    """The verify step on pooled conv_state / state / inter_ssm / conv_window (see kda_pool_desc)."""
    N, T, H, HV, K, V = p.N, p.T, p.H, p.HV, p.K, p.V
    C = 2 * H * K + HV * V
    dt = _TORCH_DT.get(p.in_dtype)
    if dt is None:
        raise KdaError(-3, "kda_conv_verify_decode_pooled")
    _check("mixed_qkv", mixed_qkv, (N, T, C), dt)
    _check("conv_weight", conv_weight, (C, 4), dt)
    _check("conv_state", conv_state, (pools.conv_state_slots, C, 3), dt)
    _check("gate", gate, (N, T, HV, K), dt)
    _check("A_log", A_log, (HV,), torch.float32)
    _check("dt_bias", dt_bias, (HV * K,), torch.float32)
    _check("beta", beta, (N, T, HV), dt)
    _check("state", state, (pools.state_slots, HV, K, V), torch.float32)
    _check("o", o, (N, T, HV, V), dt)
    _check("inter_ssm", inter_ssm, (pools.intermediate_slots, T, HV, K, V), torch.float32)
    _check("conv_window", conv_window, (pools.intermediate_slots, T, C, 3), dt)
    ptrs = [t.data_ptr() for t in (mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                                   o, inter_ssm, conv_window, workspace)]
    st = load().kda_conv_verify_decode_pooled(ctypes.byref(p), ctypes.byref(pools), *[_VP(x) for x in ptrs],
                                              workspace.numel() * workspace.element_size(), _VP(_stream(stream)))
    if st != KDA_OK:
        raise KdaError(st, "kda_conv_verify_decode_pooled")


def kda_conv_verify_decode_unfused(p: Params, pools: Optional[PoolDesc], mixed_qkv, conv_weight, conv_state, gate,
                                   A_log, dt_bias, beta, state, o, inter_ssm, conv_window, act, workspace,
                                   stream=None) -> None:
    """The step in unfused form (separate conv kernel, fp32 activations through ``act`` [N,T,C])."""
    N, T, H, HV, K, V = p.N, p.T, p.H, p.HV, p.K, p.V
    C = 2 * H * K + HV * V
    dt = _TORCH_DT.get(p.in_dtype)
    if dt is None:
        raise KdaError(-3, "kda_conv_verify_decode_unfused")
    if pools is None:
        pools = make_pools(N)
    _check("mixed_qkv", mixed_qkv, (N, T, C), dt)
    _check("conv_weight", conv_weight, (C, 4), dt)
    _check("conv_state", conv_state, (pools.conv_state_slots, C, 3), dt)
    _check("gate", gate, (N, T, HV, K), dt)
    _check("A_log", A_log, (HV,), torch.float32)
    _check("dt_bias", dt_bias, (HV * K,), torch.float32)
    _check("beta", beta, (N, T, HV), dt)
    _check("state", state, (pools.state_slots, HV, K, V), torch.float32)
    _check("o", o, (N, T, HV, V), dt)
    _check("inter_ssm", inter_ssm, (pools.intermediate_slots, T, HV, K, V), torch.float32)
    _check("conv_window", conv_window, (pools.intermediate_slots, T, C, 3), dt)
    _check("act", act, (N, T, C), torch.float32)
    ptrs = [t.data_ptr() for t in (mixed_qkv, conv_weight, conv_state, gate, A_log, dt_bias, beta, state,
                                   o, inter_ssm, conv_window, act, workspace)]
    st = load().kda_conv_verify_decode_unfused(ctypes.byref(p), ctypes.byref(pools), *[_VP(x) for x in ptrs],
                                               workspace.numel() * workspace.element_size(), _VP(_stream(stream)))
    if st != KDA_OK:
        raise KdaError(st, "kda_conv_verify_decode_unfused")


def verify_commit(p: Params, pools: PoolDesc, accepted, inter_ssm, conv_window, state, conv_state,
                  stream=None) -> None:
    """Accept step: state/conv_state rows <- the snapshots of each sequence's last accepted token."""
    N, T, H, HV, K, V = p.N, p.T, p.H, p.HV, p.K, p.V
    C = 2 * H * K + HV * V
    dt = _TORCH_DT.get(p.in_dtype)
    if dt is None:
        raise KdaError(-3, "kda_verify_commit")
    if pools is None:
        pools = make_pools(N)
    _check("accepted", accepted, (N,), torch.int32)
    _check("inter_ssm", inter_ssm, (pools.intermediate_slots, T, HV, K, V), torch.float32)
    _check("conv_window", conv_window, (pools.intermediate_slots, T, C, 3), dt)
    _check("state", state, (pools.state_slots, HV, K, V), torch.float32)
    _check("conv_state", conv_state, (pools.conv_state_slots, C, 3), dt)
    ptrs = [t.data_ptr() for t in (accepted, inter_ssm, conv_window, state, conv_state)]
    st = load().kda_verify_commit(ctypes.byref(p), ctypes.byref(pools), *[_VP(x) for x in ptrs],
                                  _VP(_stream(stream)))
    if st != KDA_OK:
        raise KdaError(st, "kda_verify_commit")


def alloc_outputs(w, device="cuda") -> Dict[str, torch.Tensor]:
    """Output buffers (o, inter_ssm, conv_window) for a ``synth.Workload``."""
    dt = w.torch_dtype
    return {
        "o": torch.empty((w.N, w.T, w.HV, w.V), dtype=dt, device=device),
        "inter_ssm": torch.empty((w.N, w.T, w.HV, w.K, w.V), dtype=torch.float32, device=device),
        "conv_window": torch.empty((w.N, w.T, w.C, 3), dtype=dt, device=device),
    }


def run(p: Params, inp: Dict[str, torch.Tensor], out: Dict[str, torch.Tensor], workspace: torch.Tensor,
        stream=None) -> None:
    """``kda_conv_verify_decode`` with inputs and outputs given as dicts (conv_state in ``inp``)."""
    kda_conv_verify_decode(p, inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"], inp["gate"],
                           inp["A_log"], inp["dt_bias"], inp["beta"], inp["state"], out["o"],
                           out["inter_ssm"], out["conv_window"], workspace, stream)
