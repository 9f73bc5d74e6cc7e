"""Every branch of the dispatch rule on grids of 129-2304 (sequence, value head) units, on
the GPU through the C ABI: one generation of whole-V workgroups in one, two or four column
groups with either store policy (129-512 units), the uncapped grid below 1024 units; value-head counts that are not powers of
two among them (HV = 12, 24, 36, 40, 48); two workgroups per CU below 1280 units at T = 3,
4, the uncapped grid at T = 1 up to 3071 units, and the stream schedule (the queue beyond
T = 8) from 1280 units at T = 2-4, from 1024 at T >= 5 and from 3072 at T = 1.

For each shape the launch AUTO picks is pinned, its results must equal those of the
32-column split bit for bit (every launch shares the K split and the partial-sum tree),
conv_window and the rolled conv_state must equal the shift-register definition bit for bit,
and o and inter_ssm of every sequence must be within max-abs 2e-3 of the float64 oracle.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), PR
description (small and large variants share one API and math; HV >= H) and Tests &
Accuracy (variants bit-identical, conv state bit-exact).
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_kda_amd as kda
import oracle
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches_all, bits, ref_bits, run_gpu, say

pytestmark = pytest.mark.gpu

# (N, T, H, HV, gate) -> the launch AUTO must pick: (tile, store policy, cap, groups, schedule)
CASES = [
    ((12, 2, 4, 12, "softplus"), (128, 1, 0, 2, 1)),    # 144 units, T = 2: two groups, streaming stores
    ((6, 5, 4, 40, "safe"), (128, 2, 0, 2, 1)),         # 240 units, odd T below 256: two groups
    ((16, 7, 16, 16, "softplus"), (128, 2, 0, 1, 1)),   # 256 units, odd T: one group, device scope
    ((32, 3, 12, 12, "safe"), (128, 2, 0, 1, 1)),       # 384 units, odd T, HV = 12
    ((8, 4, 32, 32, "safe"), (128, 1, 0, 2, 1)),        # 256 units, T = 4: two groups, streaming
    ((16, 4, 8, 24, "softplus"), (128, 1, 0, 2, 1)),    # 384 units, T = 4, HV = 24
    ((16, 6, 8, 24, "safe"), (128, 2, 0, 2, 1)),        # 384 units, T = 6: device scope
    ((8, 8, 16, 48, "softplus"), (128, 2, 0, 2, 1)),    # 384 units, T = 8, HV = 48
    ((20, 1, 8, 24, "safe"), (128, 2, 0, 1, 1)),        # 480 units, T = 1: one group
    ((24, 3, 12, 36, "softplus"), (128, 2, 0, 1, 1)),   # 864 units, T = 3: the uncapped grid
    ((40, 4, 12, 24, "safe"), (128, 2, 0, 1, 1)),       # 960 units, T = 4: the uncapped grid
    ((9, 1, 32, 32, "softplus"), (128, 2, 0, 1, 1)),    # 288 units, T = 1: one group beyond 256
    ((48, 4, 12, 24, "softplus"), (128, 2, 2, 1, 1)),   # 1152 units, T = 4: two per CU
    ((64, 4, 12, 24, "softplus"), (128, 2, 1, 1, 3)),   # 1536 units, T = 4: the stream from 1280
    ((40, 2, 16, 32, "safe"), (128, 2, 1, 1, 3)),       # 1280 units, T = 2: the stream
    ((96, 1, 8, 24, "safe"), (128, 2, 0, 1, 1)),        # 2304 units, T = 1: the uncapped grid
    ((128, 1, 16, 32, "softplus"), (128, 2, 1, 1, 3)),  # 4096 units, T = 1: the stream from 3072
    ((48, 3, 16, 48, "softplus"), (128, 2, 1, 1, 3)),   # 2304 units, T = 3: the stream, state at the start
    ((96, 2, 12, 24, "safe"), (128, 2, 1, 1, 3)),       # 2304 units, T = 2: the stream
    ((24, 6, 8, 48, "softplus"), (128, 2, 1, 1, 3)),    # 1152 units, T = 6: the stream from 1024 at T >= 5
    ((128, 9, 8, 16, "safe"), (128, 2, 1, 1, 2)),       # 2048 units, T = 9: the queue beyond T = 8
]


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    dt = torch.int16 if a.element_size() == 2 else torch.int32
    return torch.equal(a.view(dt), b.view(dt))


@pytest.mark.parametrize("shape,launch", CASES, ids=[f"N{c[0][0]}-T{c[0][1]}-H{c[0][2]}-HV{c[0][3]}" for c in CASES])
def test_bucket_launch_and_parity(shape, launch):
    N, T, H, HV, gate = shape
    w = synth.Workload(f"bucket-N{N}-T{T}-H{H}-HV{HV}", N=N, T=T, H=H, HV=HV, K=128, V=128,
                       dtype="bf16", gate=gate, seed=7000 + 10 * T + HV)
    assert tuple(kda.select_launch(kda.params_for(w)).values())[:5] == launch
    inp = synth.make_inputs(w)
    x0, cs0 = inp["mixed_qkv"].clone(), inp["conv_state"].clone()
    auto = run_gpu(w, inp, kda.VARIANT_AUTO)
    split = run_gpu(w, inp, kda.VARIANT_SMALL)
    for k in ("o", "inter_ssm", "conv_window", "conv_state"):
        assert _bits_equal(auto[k], split[k]), f"{w.name}: {k} differs between AUTO {launch} and the 32-column split"
    del split
    cw_ref, cs_ref = oracle.conv_roll(x0, cs0)
    assert np.array_equal(bits(auto["conv_window"]), ref_bits(cw_ref, w.torch_dtype)), f"{w.name}: conv_window"
    assert np.array_equal(bits(auto["conv_state"]), ref_bits(cs_ref, w.torch_dtype)), f"{w.name}: conv_state"
    err = assert_matches_all(w, inp, auto, what=w.name)
    say(f"{w.name}: launch {launch}, bit-identical to the split, all {N} sequences max-abs o={err['o']:.2e} "
        f"inter_ssm={err['inter_ssm']:.2e}")
