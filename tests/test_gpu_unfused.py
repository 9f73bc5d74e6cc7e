"""GPU parity of the unfused form of the step (separate conv kernel, activations through
HBM), the baseline that measures what fusion saves.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), PR
description: fusion removes the separate conv launch and the intermediate round trips.
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches, assert_matches_all, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def W(N, T, H, HV, K=128, V=128, dtype="bf16", gate="softplus", seed=13):
    return synth.Workload(f"unf{N}x{T}x{H}x{HV}x{K}", N=N, T=T, H=H, HV=HV, K=K, V=V, dtype=dtype, gate=gate,
                          seed=seed)


def run_unfused(w, inp, **pkw):
    say(f"[gpu] unfused {w.name} {w.dtype} {w.gate}")
    p = kda.params_for(w, **pkw)
    g = to_dev(inp)
    out = kda.alloc_outputs(w)
    for t in out.values():
        t.fill_(float("nan"))
    act = torch.empty((w.N, w.T, w.C), dtype=torch.float32, device="cuda")
    kda.kda_conv_verify_decode_unfused(p, None, g["mixed_qkv"], g["conv_weight"], g["conv_state"], g["gate"],
                                       g["A_log"], g["dt_bias"], g["beta"], g["state"], out["o"], out["inter_ssm"],
                                       out["conv_window"], act, kda.alloc_workspace(p))
    torch.cuda.synchronize()
    out["conv_state"] = g["conv_state"]
    out["act"] = act
    return out


@pytest.mark.parametrize("w", [W(3, 4, 2, 4), W(2, 2, 2, 2, K=16, V=16, dtype="f32", gate="safe"),
                               W(4, 8, 1, 2, K=64, V=64), W(5, 3, 2, 2, dtype="f32")])
def test_unfused_matches_oracle(w):
    inp = synth.make_inputs(w)
    got = run_unfused(w, inp)
    assert_matches(w, got, oracle.verify_workload(w, inp), what=f"unfused {w.name}")
    # the fp32 activations the first kernel wrote: SiLU(conv)
    act = oracle.conv_silu(inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"])
    np.testing.assert_allclose(got["act"].double().cpu().numpy(), act, rtol=1e-5, atol=1e-5)


def test_unfused_close_to_fused_at_full_size():
    """The GVA workload (N=64, T=3, H=16, HV=32) fused and unfused: identical raw copies,
    and the same arithmetic from the activations on, so o and the snapshots agree closely."""
    w = synth.WORKLOADS["gva"]
    inp = synth.make_inputs(w)
    a = run_gpu(w, inp)
    b = run_unfused(w, inp)
    assert torch.equal(a["conv_window"], b["conv_window"]) and torch.equal(a["conv_state"], b["conv_state"])
    assert (a["inter_ssm"] - b["inter_ssm"]).abs().max().item() <= 2e-3
    assert (a["o"].float() - b["o"].float()).abs().max().item() <= 2e-3
    assert_matches_all(w, inp, b, what="unfused gva")


def test_unfused_rejects_the_queue_schedule():
    """The unfused form keeps one workgroup per unit: an explicit queue or stream is refused
    before anything launches, and AUTO, which would pick the stream for the fused step, runs
    the grid."""
    w = W(128, 4, 32, 32)  # 4096 units: AUTO's stream for the fused step
    inp = synth.make_inputs(w)
    for sched in (2, 3):
        with pytest.raises(kda.KdaError):
            run_unfused(w, inp, schedule=sched)
    assert kda.select_launch(kda.params_for(w))["schedule"] == 3
    got = run_unfused(w, inp)
    assert_matches_all(w, inp, got, what="unfused, AUTO")
