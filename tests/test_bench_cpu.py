"""Host-side parts of bench.py: the multi-GPU refusal and the CPU-baseline legs (no GPU)."""
import json
import os
import subprocess
import sys

import bench
from linear_attention_decode_kda_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_legs_on_tiny_workload():
    w = synth.WORKLOADS["tiny"]
    cpu = bench.cpu_baseline(w, synth.make_inputs(w), 0.2, 2)
    json.dumps(cpu)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "tokens/s" and cpu["cores"] == 2
    assert cpu["value"] > 0 and cpu["single_thread"]["value"] > 0
    assert cpu["single_thread"]["cores"] == 1
    # the host is described: threads used, the host's CPUs and the CPU model, kept distinct
    assert cpu["threads"] == 2 and cpu["host_cores"] == os.cpu_count()
    assert 1 <= cpu["cpus_allowed"] <= cpu["host_cores"] and isinstance(cpu["cpu_model"], str)
    assert cpu["cpu_model"] == bench.cpu_model() != ""


def test_cpu_baseline_parity_readout():
    """The parity readout of the CPU-baseline leg, fed the oracle's own outputs in their
    stored dtypes (standing in for a GPU call): zero error and bit-exact conv outputs pass;
    one snapshot element off by 1e-2 and one flipped conv-cache value each fail."""
    import torch

    import oracle
    w = synth.WORKLOADS["tiny"]
    inp = synth.make_inputs(w)
    ref = oracle.verify_workload(w, inp)
    dt = w.torch_dtype

    def as_gpu():
        return {"o": torch.from_numpy(ref["o"]).to(dt), "inter_ssm": torch.from_numpy(ref["inter_ssm"]).float(),
                "conv_window": torch.from_numpy(ref["conv_window"]).to(dt),
                "conv_state": torch.from_numpy(ref["conv_state"]).to(dt)}

    par = bench.cpu_baseline(w, inp, 0.2, 2, as_gpu())["parity"]
    json.dumps(par)
    assert par["pass"] and par["sequences"] == w.N and par["tolerance"] == bench.PARITY_TOL
    assert par["conv_window_bit_exact"] and par["conv_state_bit_exact"]
    assert par["o_max_abs_err"] < 1e-6 and par["inter_ssm_max_abs_err"] < 1e-6
    bad = as_gpu()
    bad["inter_ssm"][1, 0, 1, 2, 3] += 1e-2
    par = bench.cpu_baseline(w, inp, 0.2, 2, bad)["parity"]
    assert not par["pass"] and par["inter_ssm_max_abs_err"] > bench.PARITY_TOL and par["conv_state_bit_exact"]
    bad = as_gpu()
    bad["conv_state"][0, 5, 1] = -bad["conv_state"][0, 5, 1] - 1
    par = bench.cpu_baseline(w, inp, 0.2, 2, bad)["parity"]
    assert not par["pass"] and not par["conv_state_bit_exact"] and par["conv_window_bit_exact"]


def test_host_threads_bounds(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "64")
    assert bench.host_threads() == 16
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_threads() == 3
    monkeypatch.setenv("OMP_NUM_THREADS", "junk")
    assert 1 <= bench.host_threads() <= 16


def test_sweep_launch_names_round_trip():
    """Every launch the dispatch sweep times, given as overrides, is reported back by the
    library's launch selection under the same name, so that a sweep table can find the
    launch the rule picks among the timed ones (no GPU: host-only selection)."""
    import linear_attention_decode_kda_amd as kda
    launches = bench.sweep_launches()
    assert "stream s2 p1" in launches and "stream s2 p2" in launches and len(launches) == 29
    for name, kw in launches.items():
        ln = kda.select_launch(kda.make_params(64, 4, 16, 32, 128, 128, **kw))
        assert bench.launch_name(ln) == name, (name, ln)
    # the rule's own picks on the named workloads carry sweep names too
    for wl, want in (("small_batch", "grid g1 s1 o2"), ("gva", "stream s2 p2"), ("large_batch", "stream s2 p2"),
                     ("max_bandwidth", "stream s2 p1")):
        assert bench.launch_name(kda.select_launch(kda.params_for(synth.WORKLOADS[wl]))) == want, wl
