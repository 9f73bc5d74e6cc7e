"""The library driven by a plain C program, linear_attention_decode_kda_amd/examples/verify_from_c.c
(built by build(): the header compiled as C11 with gcc). The program allocates its own device
buffers with hipMalloc, zeroes a workspace with kda_workspace_reset and makes one
kda_conv_verify_decode call on a stream of its own; no Python or torch runs in the process
that calls the library. Inputs reach it as raw arrays in the header's layouts and its outputs
come back the same way; the GPU test compares them with the float64 oracle on every sequence
(conv_window and the rolled conv_state bit-exact, o and inter_ssm within 2e-3).

The C program starts as a child process; this process itself never touches the GPU.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

from gpu_util import assert_matches_all, say
from linear_attention_decode_kda_amd import build as kbuild
from linear_attention_decode_kda_amd import synth

ORDER = ("mixed_qkv", "conv_weight", "conv_state", "gate", "A_log", "dt_bias", "beta", "state")
CASES = [
    synth.WORKLOADS["tiny"],                                                # fp32, K = V = 16
    synth.WORKLOADS["tiny"].with_(dtype="bf16", T=3),
    synth.Workload("c_caller_gva", 3, 4, 2, 4, 128, 128, "bf16", "safe", 71),  # two value heads per q/k head
    synth.WORKLOADS["small_batch"],                                         # 512 units, the full config
]


def _args(w, d):
    return [kbuild.EXAMPLE, str(d), *map(str, (w.N, w.T, w.H, w.HV, w.K, w.V)),
            "1" if w.dtype == "bf16" else "0", "1" if w.gate == "safe" else "0"]


def test_c_caller_is_built_and_checks_its_arguments(tmp_path):
    """No GPU: the program is built, prints its usage on bad arguments, rejects shapes and
    flags the library's validation rejects, and stops on a missing input file before any HIP
    call."""
    assert os.path.exists(kbuild.EXAMPLE), f"{kbuild.EXAMPLE} is not built; run __graft_entry__.build()"
    r = subprocess.run([kbuild.EXAMPLE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    r = subprocess.run(_args(synth.WORKLOADS["tiny"], tmp_path), capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "cannot open" in r.stderr and "mixed_qkv.bin" in r.stderr
    # shapes and flags the library rejects stop before any file is read
    for bad in (synth.WORKLOADS["tiny"].with_(HV=3), synth.WORKLOADS["tiny"].with_(N=-1),
                synth.WORKLOADS["tiny"].with_(K=8, V=8)):
        r = subprocess.run(_args(bad, tmp_path), capture_output=True, text=True, timeout=60)
        assert r.returncode == 2 and "invalid parameters" in r.stderr, (bad, r.stderr)
    r = subprocess.run(_args(synth.WORKLOADS["tiny"], tmp_path)[:-1] + ["7"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2 and "must be 0 or 1" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("w", CASES, ids=[f"{w.name}-{w.dtype}-{w.gate}-T{w.T}" for w in CASES])
def test_c_caller_matches_oracle(w, tmp_path):
    assert os.path.exists(kbuild.EXAMPLE), f"{kbuild.EXAMPLE} is not built; run __graft_entry__.build()"
    inp = synth.make_inputs(w)
    for k in ORDER:
        inp[k].contiguous().view(torch.uint8).numpy().tofile(tmp_path / f"{k}.bin")
    say(f"[gpu] C caller {w.name} N={w.N} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V} {w.dtype} {w.gate}")
    r = subprocess.run(_args(w, tmp_path), capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "verify_from_c ok" in r.stdout, r.stdout + r.stderr

    def load(name, dtype, shape):
        raw = np.fromfile(tmp_path / f"{name}.bin", dtype=np.uint8)
        return torch.from_numpy(raw).view(dtype).reshape(shape)

    dt, C = w.torch_dtype, w.C
    got = {"o": load("o", dt, (w.N, w.T, w.HV, w.V)),
           "inter_ssm": load("inter_ssm", torch.float32, (w.N, w.T, w.HV, w.K, w.V)),
           "conv_window": load("conv_window", dt, (w.N, w.T, C, 3)),
           "conv_state": load("conv_state_out", dt, (w.N, C, 3))}
    assert_matches_all(w, inp, got, what=f"C caller {w.name}")
