"""Benchmark of the fused causal-conv1d + KDA multi-token verify step on one MI355X.

One step = one fused verify call (conv + SiLU, l2norm, gate, beta, gated delta rule
over T tokens, snapshots, conv window and rolled cache) over the whole batch, with
inputs already resident in HBM. Prints one JSON line:

  value      verify tokens/s = N*T / (time per call)
  roofline   algorithmic HBM bytes per call / average kernel duration (HIP events on
             the launch stream), against the MI355X HBM peak of 8 TB/s
  cpu_baseline  the float64 oracle on a bounded sample of the same workload, 1 core

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large_batch]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("linear_attention_decode_kda_amd/csrc/kda_verify.hip", "include/kda_verify.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, variant: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("source_hash") != source_hash() or doc.get("variant") != variant:
        return None
    return doc.get("hbm_bytes_per_call")


def first_sequences(inp, n):
    """The inputs of sequences 0..n-1 (per-sequence tensors sliced, shared ones kept)."""
    per_seq = ("mixed_qkv", "conv_state", "gate", "beta", "state")
    return {k: (v[:n].contiguous() if k in per_seq else v) for k, v in inp.items()}


def cpu_baseline(w, inp_cpu, budget_s: float):
    """The oracle as it is (float64, sequential C, one thread) on the first n sequences
    of the same inputs, n chosen from a one-sequence probe to take about budget_s."""
    import oracle

    oracle.load()
    t0 = time.perf_counter()
    oracle.verify_workload(w.with_(N=1), first_sequences(inp_cpu, 1))
    t1 = time.perf_counter() - t0
    n = int(max(1, min(w.N, budget_s / max(t1, 1e-6))))
    sample = first_sequences(inp_cpu, n)
    t0 = time.perf_counter()
    oracle.verify_workload(w.with_(N=n), sample)
    el = time.perf_counter() - t0
    return {
        "value": n * w.T / el,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {n} of {w.N} sequences ({n * w.HV} of {w.units} (sequence, value-head) units), "
                  f"all T={w.T} tokens, same inputs; {el:.1f} s on one host thread",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_batch")
    ap.add_argument("--variant", default="auto", choices=["auto", "small", "large"])
    ap.add_argument("--op", default="verify", choices=["verify", "verify_pooled", "commit"],
                    help="verify (the headline), verify on pooled buffers with scattered rows, or the accept step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the fused verify step has no cross-GPU exchange, "
              "and multi-GPU runs are not part of this benchmark (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 28  # 2**28 fp32 = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return

    w = synth.WORKLOADS[args.workload]
    variant = {"auto": kda.VARIANT_AUTO, "small": kda.VARIANT_SMALL, "large": kda.VARIANT_LARGE}[args.variant]
    p = kda.params_for(w, variant=variant)
    resolved = {kda.VARIANT_SMALL: "small", kda.VARIANT_LARGE: "large"}[kda.select_variant(p)]
    print(f"[bench] workload={w.name} N={w.N} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V} "
          f"{w.dtype} {w.gate} variant={resolved}", file=sys.stderr, flush=True)
    inp_cpu = synth.make_inputs(w)
    inp = {k: v.to(dev) for k, v in inp_cpu.items()}
    out = kda.alloc_outputs(w, dev)
    ws = kda.alloc_workspace(p, dev)
    stream = torch.cuda.current_stream()

    if args.op == "verify":
        def step():
            kda.run(p, inp, out, ws, stream)
        b_alg = synth.algorithmic_bytes(w)
    else:
        # pools twice the batch, sequence rows scattered by a seeded permutation
        g = torch.Generator().manual_seed(w.seed)
        slots = 2 * w.N
        idx = {k: torch.randperm(slots, generator=g)[: w.N].to(torch.int32).to(dev)
               for k in ("cs", "st", "in")}
        pools = kda.make_pools(w.N, idx["cs"], idx["st"], idx["in"], slots, slots, slots)
        cs_pool = torch.zeros((slots, w.C, 3), dtype=w.torch_dtype, device=dev)
        st_pool = torch.zeros((slots, w.HV, w.K, w.V), dtype=torch.float32, device=dev)
        cs_pool[idx["cs"].long()] = inp["conv_state"]
        st_pool[idx["st"].long()] = inp["state"]
        is_pool = torch.zeros((slots, w.T, w.HV, w.K, w.V), dtype=torch.float32, device=dev)
        cw_pool = torch.zeros((slots, w.T, w.C, 3), dtype=w.torch_dtype, device=dev)

        def verify_pooled():
            kda.kda_conv_verify_decode_pooled(p, pools, inp["mixed_qkv"], inp["conv_weight"], cs_pool, inp["gate"],
                                              inp["A_log"], inp["dt_bias"], inp["beta"], st_pool, out["o"],
                                              is_pool, cw_pool, ws, stream)
        if args.op == "verify_pooled":
            step = verify_pooled
            b_alg = synth.algorithmic_bytes(w) + 3 * 4 * w.N
        else:
            verify_pooled()
            acc = (torch.arange(w.N, dtype=torch.int32) % w.T + 1).to(dev)

            def step():
                kda.verify_commit(p, pools, acc, is_pool, cw_pool, st_pool, cs_pool, stream)
            s_in = 2 if w.dtype == "bf16" else 4
            b_alg = w.N * (2 * 4 * w.HV * w.K * w.V + 2 * 3 * s_in * w.C) + 4 * 4 * w.N

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    region_ms = ev[0][0].elapsed_time(ev[-1][1])
    avg_kernel_s = sum(kern_ms) / len(kern_ms) / 1e3
    ms_per_step = wall * 1e3 / K
    tokens = w.N * w.T
    achieved = b_alg / avg_kernel_s / 1e9
    print(f"[bench] {K} steps: wall {ms_per_step:.4f} ms/step, events {region_ms / K:.4f} ms/step, "
          f"kernel avg {avg_kernel_s * 1e3:.4f} ms min {min(kern_ms):.4f} max {max(kern_ms):.4f}; "
          f"{achieved:.0f} GB/s = {100 * achieved / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f}",
          file=sys.stderr, flush=True)

    traffic = measured_traffic(w.name, resolved) if args.op == "verify" else None
    cpu = None
    if not args.no_cpu_baseline and args.op == "verify":
        print("[bench] timing the float64 oracle on a bounded sample (cpu_baseline)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp_cpu, args.cpu_budget)

    line = {
        "metric": "verify tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: N={w.N} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V}",
            "op": args.op,
            "N": w.N, "T": w.T, "H": w.H, "HV": w.HV, "K": w.K, "V": w.V,
            "in_dtype": w.dtype, "state_dtype": "f32", "gate": w.gate, "variant": resolved,
            "algorithmic_bytes_per_call": b_alg,
            "hbm_gbps": achieved, "pct_of_hbm_peak": 100 * achieved / HBM_PEAK_GBPS,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
