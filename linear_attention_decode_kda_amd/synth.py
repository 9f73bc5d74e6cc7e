"""Seeded synthetic inputs and the workload table for the fused conv1d + KDA verify step.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no arithmetic of the method: it only draws random tensors of
the right shapes and dtypes, and it names the workloads.

Recipe (fixed, so that every caller sees the same bits whatever its thread count):

* Tensors j = 0..7, in this order, all drawn in float32: mixed_qkv ~ N(0, 1),
  conv_weight ~ N(0, 0.5), conv_state ~ N(0, 1), gate ~ N(0, 1), A_log ~ U(0, 1),
  dt_bias ~ N(0, 0.1), beta ~ N(0, 1), state ~ N(0, 0.1). The second argument of
  N(., .) is read as the standard deviation.
* Each tensor is filled in chunks of 2**24 elements (row-major order); chunk i of
  tensor j comes from its own CPU ``torch.Generator`` seeded with
  (seed << 32) ^ (j << 24) ^ i. Chunks are drawn on a thread pool.
* mixed_qkv, conv_weight, conv_state, gate and beta are then rounded to the input
  dtype (bf16 or fp32); A_log, dt_bias and state stay fp32.

The channel layout of ``mixed_qkv`` is q (H*K) | k (H*K) | v (HV*V), head-major inside
each block, the packed pre-convolution activations described on the cuLA pull request
page "[KDA] Fuse causal conv1d into MTP verify decode #107" (PR description).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    dtype: str  # "f32" | "bf16": dtype of mixed_qkv, conv_weight, conv_state, gate, beta, o
    gate: str  # "softplus" | "safe"
    seed: int

    @property
    def C(self) -> int:
        return 2 * self.H * self.K + self.HV * self.V

    @property
    def units(self) -> int:
        return self.N * self.HV

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch_dtype(self.dtype)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


# The five workloads: sizes, input dtype and gate form of each.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny", N=2, T=2, H=2, HV=2, K=16, V=16, dtype="f32", gate="softplus", seed=1000),
        Workload("small_batch", N=32, T=4, H=16, HV=16, K=128, V=128, dtype="bf16", gate="safe", seed=1001),
        Workload("gva", N=64, T=3, H=16, HV=32, K=128, V=128, dtype="bf16", gate="softplus", seed=1002),
        Workload("large_batch", N=256, T=4, H=32, HV=32, K=128, V=128, dtype="bf16", gate="softplus", seed=1003),
        Workload("max_bandwidth", N=512, T=8, H=16, HV=64, K=128, V=128, dtype="bf16", gate="safe", seed=1004),
    )
}

# Default numeric parameters of the step (the same defaults the C-ABI documents).
LOWER_BOUND = -5.0
SOFTPLUS_BETA = 1.0
SOFTPLUS_THRESHOLD = 20.0
L2NORM_EPS = 1e-6

INPUT_NAMES = ("mixed_qkv", "conv_weight", "conv_state", "gate", "A_log", "dt_bias", "beta", "state")


CHUNK = 1 << 24


def _draw(shape, seed: int, j: int, kind: str, scale: float, pool: ThreadPoolExecutor) -> torch.Tensor:
    n = 1
    for d in shape:
        n *= d
    flat = torch.empty(n, dtype=torch.float32)

    def fill(i: int) -> None:
        g = torch.Generator(device="cpu")
        g.manual_seed((seed << 32) ^ (j << 24) ^ i)
        part = flat[i * CHUNK:min(n, (i + 1) * CHUNK)]
        if kind == "normal":
            torch.randn(part.numel(), generator=g, out=part)
        else:
            torch.rand(part.numel(), generator=g, out=part)

    list(pool.map(fill, range((n + CHUNK - 1) // CHUNK)))
    if scale != 1.0:
        flat.mul_(scale)
    return flat.view(shape)


def make_inputs(w: Workload, seed: int | None = None) -> Dict[str, torch.Tensor]:
    """Draw one set of inputs for workload ``w`` on the CPU (see the module recipe)."""
    seed = w.seed if seed is None else seed
    N, T, HV, K, V, C = w.N, w.T, w.HV, w.K, w.V, w.C
    dt = w.torch_dtype
    spec = [
        ("mixed_qkv", (N, T, C), "normal", 1.0, dt),
        ("conv_weight", (C, 4), "normal", 0.5, dt),
        ("conv_state", (N, C, 3), "normal", 1.0, dt),
        ("gate", (N, T, HV, K), "normal", 1.0, dt),
        ("A_log", (HV,), "uniform", 1.0, torch.float32),
        ("dt_bias", (HV * K,), "normal", 0.1, torch.float32),
        ("beta", (N, T, HV), "normal", 1.0, dt),
        ("state", (N, HV, K, V), "normal", 0.1, torch.float32),
    ]
    out = {}
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as pool:
        for j, (name, shape, kind, scale, odt) in enumerate(spec):
            t = _draw(shape, seed, j, kind, scale, pool)
            out[name] = t if odt == torch.float32 else t.to(odt)
    return out


def output_shapes(w: Workload) -> Dict[str, tuple]:
    """Shapes of the buffers the step writes."""
    return {
        "o": (w.N, w.T, w.HV, w.V),
        "inter_ssm": (w.N, w.T, w.HV, w.K, w.V),
        "conv_window": (w.N, w.T, w.C, 3),
        "conv_state": (w.N, w.C, 3),
    }


def algorithmic_bytes(w: Workload) -> int:
    """Bytes one call must move at minimum (each input read once, each output written once).

    q/k channels are counted once per sequence, not once per value head.
    """
    s = 2 if w.dtype == "bf16" else 4
    N, T, HV, K, V, C = w.N, w.T, w.HV, w.K, w.V, w.C
    b = 0
    b += 4 * N * HV * K * V  # state read
    b += 4 * N * T * HV * K * V  # inter_ssm write
    b += s * N * T * C  # mixed_qkv read
    b += s * 4 * C  # conv_weight read
    b += 2 * s * 3 * N * C  # conv_state read + write
    b += s * 3 * N * T * C  # conv_window write
    b += s * N * T * HV * K + 4 * HV + 4 * HV * K  # gate, A_log, dt_bias
    b += s * N * T * HV  # beta
    b += s * N * T * HV * V  # o
    return b
