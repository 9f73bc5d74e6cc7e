"""Helpers shared by the GPU tests: run the HIP path, compare it with the oracle."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

import linear_attention_decode_kda_amd as kda
from linear_attention_decode_kda_amd import synth

TOL = 2e-3  # max-abs error allowed on o and inter_ssm (fp32 state, bf16 or fp32 inputs)


def say(msg: str) -> None:
    """Name the case before a GPU step so a failure report says what ran."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(inp: Dict[str, torch.Tensor], dev="cuda") -> Dict[str, torch.Tensor]:
    return {k: v.to(dev).contiguous() for k, v in inp.items()}


def run_gpu(w: synth.Workload, inp: Dict[str, torch.Tensor], variant: int = kda.VARIANT_AUTO,
            poison: bool = True, **pkw) -> Dict[str, torch.Tensor]:
    """One call on the GPU; returns GPU tensors o, inter_ssm, conv_window and the rolled conv_state."""
    say(f"[gpu] {w.name} N={w.N} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V} {w.dtype} {w.gate} variant={variant}")
    p = kda.params_for(w, variant=variant, **pkw)
    g = to_dev(inp)
    out = kda.alloc_outputs(w)
    if poison:
        for t in out.values():
            t.fill_(float("nan"))
    ws = kda.alloc_workspace(p)
    kda.run(p, g, out, ws)
    torch.cuda.synchronize()
    out["conv_state"] = g["conv_state"]
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def ref_bits(a: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Bits of oracle float64 values that are exact copies of stored inputs."""
    return bits(torch.from_numpy(a).to(dtype))


def assert_matches(w: synth.Workload, got: Dict[str, torch.Tensor], ref: Dict[str, np.ndarray],
                   n_index: Optional[np.ndarray] = None, what: str = "") -> Dict[str, float]:
    """conv_window / conv_state bit-exact, o / inter_ssm within TOL, no NaN anywhere.

    ``n_index`` selects the sequences of ``got`` that ``ref`` covers (the oracle ran on a slice).
    """
    sel = (lambda t: t) if n_index is None else (lambda t: t[torch.as_tensor(n_index, device=t.device)])
    dt = w.torch_dtype
    cw, cs = sel(got["conv_window"]), sel(got["conv_state"])
    assert np.array_equal(bits(cw), ref_bits(ref["conv_window"], dt)), f"{what}: conv_window not bit-exact"
    assert np.array_equal(bits(cs), ref_bits(ref["conv_state"], dt)), f"{what}: conv_state not bit-exact"
    o = sel(got["o"]).float().cpu().numpy()
    s = sel(got["inter_ssm"]).cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s)), f"{what}: non-finite output"
    eo = float(np.abs(o - ref["o"]).max())
    es = float(np.abs(s - ref["inter_ssm"]).max())
    assert eo <= TOL, f"{what}: o max-abs error {eo:.3g} > {TOL}"
    assert es <= TOL, f"{what}: inter_ssm max-abs error {es:.3g} > {TOL}"
    return {"o": eo, "inter_ssm": es}


def slice_inputs(inp: Dict[str, torch.Tensor], idx) -> Dict[str, torch.Tensor]:
    """Inputs of the sequences ``idx`` (per-sequence tensors sliced, shared ones kept)."""
    per_seq = ("mixed_qkv", "conv_state", "gate", "beta", "state")
    ix = torch.as_tensor(idx)
    return {k: (v[ix].contiguous() if k in per_seq else v) for k, v in inp.items()}


PER_SEQ = ("mixed_qkv", "conv_state", "gate", "beta", "state")


def host_threads() -> int:
    """Worker threads for the oracle: the host's CPUs, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def assert_matches_all(w: synth.Workload, inp: Dict[str, torch.Tensor], got: Dict[str, torch.Tensor],
                       chunk: int = 4, what: str = "") -> Dict[str, float]:
    """Every sequence of ``got`` against the float64 oracle, in slices of ``chunk`` sequences.

    ``inp`` holds the CPU inputs of the call (conv_state before it was rolled); ``got`` the
    GPU outputs (o, inter_ssm, conv_window and the rolled conv_state). Each slice runs the
    oracle on its own host thread (the oracle is plain C called through ctypes, which
    releases the GIL) and copies only its own sequences back from the GPU, so host memory
    stays bounded by the slices in flight even when inter_ssm is many GiB. Returns the
    largest max-abs errors over all slices and the relative RMS errors over the whole
    batch: of inter_ssm, and of o against the oracle's o rounded to the output dtype.
    """
    import oracle

    oracle.load()
    N = w.N

    def one(a: int):
        b = min(N, a + chunk)
        part = {k: (v[a:b].contiguous() if k in PER_SEQ else v) for k, v in inp.items()}
        ref = oracle.verify_workload(w.with_(N=b - a), part)
        sl = {k: got[k][a:b] for k in ("o", "inter_ssm", "conv_window", "conv_state")}
        e = assert_matches(w.with_(N=b - a), sl, ref, what=f"{what} sequences {a}..{b - 1}")
        o = sl["o"].float().cpu().numpy().astype(np.float64)
        o_ref = torch.from_numpy(ref["o"]).to(w.torch_dtype).double().numpy()
        s = sl["inter_ssm"].cpu().numpy().astype(np.float64)
        sums = (float(np.sum((o - o_ref) ** 2)), float(np.sum(o_ref ** 2)),
                float(np.sum((s - ref["inter_ssm"]) ** 2)), float(np.sum(ref["inter_ssm"] ** 2)))
        return e, sums

    errs = {"o": 0.0, "inter_ssm": 0.0}
    tot = [0.0, 0.0, 0.0, 0.0]
    with ThreadPoolExecutor(host_threads()) as ex:
        for e, sums in ex.map(one, range(0, N, chunk)):
            errs = {k: max(errs[k], e[k]) for k in errs}
            tot = [x + y for x, y in zip(tot, sums)]
    errs["rel_rmse_o"] = float(np.sqrt(tot[0] / tot[1])) if tot[1] > 0 else 0.0
    errs["rel_rmse_inter_ssm"] = float(np.sqrt(tot[2] / tot[3])) if tot[3] > 0 else 0.0
    return errs


def bit_view(t: torch.Tensor) -> torch.Tensor:
    """The raw bits of a GPU tensor as integers of its element width."""
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def checksums(t: torch.Tensor, row: int) -> torch.Tensor:
    """Per-row sums of the raw bits of ``t`` (rows of ``row`` elements, on the GPU), taken
    as 64-bit words (wrapping): a positional fingerprint that a change of any one element's
    bits alters, computed in one read with no temporary copy of ``t``. ``row`` elements
    must span a multiple of 8 bytes."""
    assert (row * t.element_size()) % 8 == 0 and t.is_contiguous()
    return t.reshape(-1).view(torch.int64).reshape(-1, row * t.element_size() // 8).sum(dim=1)
