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


def test_host_threads_bounds(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "64")
    assert bench.host_threads() == 16
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_threads() == 3
    monkeypatch.setenv("OMP_NUM_THREADS", "junk")
    assert 1 <= bench.host_threads() <= 16


def test_timeline_instrumentation_applies_to_the_kernel_source():
    """The timeline tool patches the current kernel source (sixteen stamps per unit); a
    kernel edit that moves one of its anchors must fail here, not on the GPU."""
    from linear_attention_decode_kda_amd import build as b
    from linear_attention_decode_kda_amd import timeline

    with open(b.SRC) as f:
        src = timeline._instrument(f.read())
    for q in range(15):
        assert f"st_[{q}]" in src, q
    assert "kda_timeline_set_stamps" in src and "a.stamps = g_stamps;" in src
