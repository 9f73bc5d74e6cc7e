"""Seeded random shapes and launch overrides against the float64 oracle.

Two draws, fixed seeds: general shapes (K = V = 16, 64, 128; one to four value heads per q/k
head; T up to 16; bf16 and fp32 inputs; both gates) with random tile, store, cap, column-group,
schedule, unit-order and prefetch overrides on K = V = 128; and shapes on the queue and the
stream (every store policy and state prefetch point). Override combinations the library
rejects are dropped when the list is drawn (host-side validation, no GPU). Every case is
compared with the oracle on every sequence: conv_window and conv_state bit-exact, o and
inter_ssm within 2e-3 max-abs.
"""
import random

import pytest

import linear_attention_decode_kda_amd as kda
from linear_attention_decode_kda_amd import synth
from gpu_util import assert_matches_all, run_gpu

pytestmark = pytest.mark.gpu


def _accepted(w, kw):
    try:
        kda.select_launch(kda.params_for(w, **kw))
        return True
    except kda.KdaError:
        return False


def _general(seed=7, draws=60):
    rng, out = random.Random(seed), []
    for i in range(draws):
        K = rng.choice([16, 64, 128, 128, 128])
        H = rng.choice([1, 2, 3, 4, 8])
        g = rng.choice([1, 1, 2, 3, 4])
        T = rng.choice([1, 2, 3, 4, 5, 6, 8, 9, 12, 16])
        N = rng.randint(1, 48)
        dtype = rng.choice(["bf16", "bf16", "f32"])
        gate = rng.choice(["softplus", "safe"])
        w = synth.Workload(f"rand{i}", N=N, T=T, H=H, HV=H * g, K=K, V=K, dtype=dtype, gate=gate, seed=5000 + i)
        kw = {}
        if K == 128 and rng.random() < 0.7:
            kw = dict(schedule=rng.choice([0, 1, 2, 3]), store_policy=rng.choice([0, 1, 2]),
                      max_wg_per_cu=rng.choice([0, 1, 2, 4, 8]), column_groups=rng.choice([0, 1, 2, 4]),
                      unit_order=rng.choice([0, 1, 2]), prefetch=rng.choice([0, 1, 2]),
                      tile_columns=rng.choice([0, 0, 32, 64, 128]))
        if _accepted(w, kw):
            out.append((w, kw))
    return out


def _queue_and_stream(seed=11, draws=40):
    rng, out = random.Random(seed), []
    for i in range(draws):
        H = rng.choice([1, 2, 3, 4, 5, 8, 16])
        g = rng.choice([1, 1, 2, 3, 4])
        sched = rng.choice([2, 3, 3])
        T = rng.choice([1, 2, 3, 4, 5, 6, 7, 8] + ([9, 12, 16] if sched == 2 else []))
        N = rng.randint(1, 64)
        dtype = rng.choice(["bf16", "bf16", "f32"])
        if dtype == "f32" and T > 8:
            dtype = "bf16"
        gate = rng.choice(["softplus", "safe"])
        w = synth.Workload(f"sched{i}", N=N, T=T, H=H, HV=H * g, K=128, V=128, dtype=dtype, gate=gate,
                           seed=7000 + i)
        kw = dict(schedule=sched, store_policy=rng.choice([0, 1, 2]), prefetch=rng.choice([0, 1, 2]))
        if sched == 2:
            kw["max_wg_per_cu"] = rng.choice([0, 1, 2])
        if _accepted(w, kw):
            out.append((w, kw))
    return out


CASES = _general() + _queue_and_stream()


@pytest.mark.parametrize("w,kw", CASES,
                         ids=[f"{w.name}-N{w.N}-T{w.T}-H{w.H}-HV{w.HV}-K{w.K}-{w.dtype}-{w.gate}" for w, kw in CASES])
def test_random_shape_matches_oracle(w, kw):
    inp = synth.make_inputs(w)
    got = run_gpu(w, inp, **kw)
    assert_matches_all(w, inp, got, what=f"{w.name} {kw}")
