"""Benchmark of the fused causal-conv1d + KDA multi-token verify step on one MI355X.

One step = one fused verify call (conv + SiLU, l2norm, gate, beta, gated delta rule
over T tokens, snapshots, conv window and rolled cache) over the whole batch, with
inputs already resident in HBM. Prints one JSON line:

  value      verify tokens/s = N*T / (time per call)
  roofline   algorithmic HBM bytes per call / average kernel duration (HIP events on
             the launch stream), against the MI355X HBM peak of 8 TB/s
  cpu_baseline  the float64 oracle on bounded samples of the same workload, on all host
                threads (sequence slices) and on one thread

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


def measured_traffic(workload: str, variant: str, launch: dict):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source and launch configuration; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("source_hash") != source_hash() or doc.get("variant") != variant or doc.get("launch") != launch:
        return None
    return doc.get("hbm_bytes_per_call")


def first_sequences(inp, n):
    """The inputs of sequences 0..n-1 (per-sequence tensors sliced, shared ones kept)."""
    per_seq = ("mixed_qkv", "conv_state", "gate", "beta", "state")
    return {k: (v[:n].contiguous() if k in per_seq else v) for k, v in inp.items()}


def device_copy_gbps(nbytes: int, dev) -> float:
    """Context for the roofline: a plain device-to-device copy moving the same number of
    bytes (reads nbytes / 2, writes nbytes / 2), in GB/s, median of 10 timed copies."""
    import torch
    n = max(1, nbytes // 8)  # float32 elements read (and written)
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[5]
    del src, dst
    return 8 * n / (ms * 1e-3) / 1e9


def host_threads() -> int:
    """Host threads for the all-core oracle leg: OMP_NUM_THREADS when set, else the CPU
    count, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_description(threads: int) -> dict:
    """What the CPU baseline ran on: the oracle's worker threads, the host's logical CPUs
    (os.cpu_count), the CPUs this process may run on (its affinity mask) and the CPU model."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return {"threads": threads, "host_cores": os.cpu_count() or 1, "cpus_allowed": allowed,
            "cpu_model": cpu_model()}


def cpu_baseline(w, inp_cpu, budget_s: float, threads: int):
    """The oracle as it is (float64, sequential C) on bounded samples of the same inputs,
    run on slices of 4 sequences: (1) on one host thread over the first n sequences, n
    chosen from a one-slice probe to take about budget_s / 2; (2) on all `threads` host
    threads, each running the oracle on its own slices (ctypes releases the GIL), over as
    many of the batch's sequences as fit in about budget_s / 2 (short samples repeated)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.load()
    chunk = 4
    per_seq = ("mixed_qkv", "conv_state", "gate", "beta", "state")

    def run_slice(ab):
        a, b = ab
        part = {k: (v[a:b].contiguous() if k in per_seq else v) for k, v in inp_cpu.items()}
        oracle.verify_workload(w.with_(N=b - a), part)
        return b - a

    def slices(n, passes=1):
        return [(a, min(a + chunk, n)) for a in range(0, n, chunk)] * passes

    t0 = time.perf_counter()
    run_slice((0, min(chunk, w.N)))
    probe = (time.perf_counter() - t0) / min(chunk, w.N)  # seconds per sequence
    n = int(max(1, min(w.N, 0.5 * budget_s / max(probe, 1e-6))))
    passes1 = int(max(1, min(20, round(0.5 * budget_s / max(n * probe, 1e-6)))))
    t0 = time.perf_counter()
    done1 = sum(run_slice(ab) for ab in slices(n, passes1))
    el = time.perf_counter() - t0
    single = {
        "value": done1 * w.T / el, "unit": "tokens/s", "cores": 1,
        "sample": f"first {n} of {w.N} sequences ({n * w.HV} of {w.units} (sequence, value-head) units), "
                  f"all T={w.T} tokens, {passes1} pass(es), slices of {chunk} sequences; {el:.1f} s on one "
                  f"host thread",
    }

    seq_rate = threads * done1 / max(el, 1e-6)  # expected sequences/s on all threads
    n_mt = int(min(w.N, max(threads * chunk, 0.5 * budget_s * seq_rate)))
    passes = int(max(1, min(20, round(0.5 * budget_s * seq_rate / n_mt))))
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        done = sum(ex.map(run_slice, slices(n_mt, passes)))
        el_mt = time.perf_counter() - t0
    return {
        "value": done * w.T / el_mt,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        **host_description(threads),
        "role": "a baseline for context, not the target",
        "sample": f"first {n_mt} of {w.N} sequences ({n_mt * w.HV} of {w.units} (sequence, value-head) units), "
                  f"all T={w.T} tokens, same inputs, {passes} pass(es), in slices of {chunk} sequences over "
                  f"{threads} host threads; {el_mt:.1f} s",
        "single_thread": single,
    }


def sweep(out_path: str, quick: bool = False, hs=None, heads_per_qk: int = 1, ts=None, units=None) -> None:
    """H = HV x T x N sweep over every tile width, snapshot store policy and workgroups-per-CU
    cap on the grid schedule, whole-V workgroups in 2 or 4 column groups on the uncapped grid
    and in 2 at one per CU, and the queue schedule of whole-V workgroups at one per CU in 1, 2 or 4 column groups
    (K = V = 128, bf16, softplus). Buffer sets are rotated so that
    at least 1 GiB is touched between reuses (small shapes would otherwise run from the
    256 MB last-level cache). A cap is timed only where the grid has more workgroups than
    the cap lets run at once, the queue only where there are more units than CUs.
    heads_per_qk > 1 gives each q/k head that many value heads (HV = heads_per_qk H); units =
    (lo, hi) keeps only the shapes with lo <= N HV <= hi. Writes one JSON object per shape to
    out_path and prints a summary line."""
    import torch

    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    dev = torch.device("cuda:0")
    Hs = tuple(hs) if hs else (8, 32) if quick else (8, 16, 32, 64)
    Ts = tuple(ts) if ts else (2, 4, 8) if quick else (1, 2, 4, 6, 8)
    Ns = (1, 8, 64, 256) if quick else (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)
    combos = [(t, pol, occ, 1, 1) for t in (32, 64, 128) for pol in (1, 2) for occ in (8, 6, 4, 2, 1)]
    combos += [(128, pol, 8, g, 1) for pol in (1, 2) for g in (2, 4)]
    combos += [(128, pol, 1, 2, 1) for pol in (1, 2)]
    combos += [(128, pol, 1, g, 2) for pol in (1, 2) for g in (1, 2, 4)]
    rows = []
    with open(out_path, "w") as f:
        for H in Hs:
            for T in Ts:
                for N in Ns:
                    HV = heads_per_qk * H
                    if units and not units[0] <= N * HV <= units[1]:
                        continue
                    w = synth.Workload(f"sweep", N=N, T=T, H=H, HV=HV, K=128, V=128, dtype="bf16",
                                       gate="softplus", seed=1)
                    b_alg = synth.algorithmic_bytes(w)
                    nset = max(1, min(16, (1 << 30) // b_alg + 1))
                    sets = []
                    for _ in range(nset):
                        inp = {
                            "mixed_qkv": torch.randn(N, T, w.C, device=dev).to(torch.bfloat16),
                            "conv_weight": (torch.randn(w.C, 4, device=dev) * 0.5).to(torch.bfloat16),
                            "conv_state": torch.randn(N, w.C, 3, device=dev).to(torch.bfloat16),
                            "gate": torch.randn(N, T, HV, 128, device=dev).to(torch.bfloat16),
                            "A_log": torch.rand(HV, device=dev),
                            "dt_bias": torch.randn(HV * 128, device=dev) * 0.1,
                            "beta": torch.randn(N, T, HV, device=dev).to(torch.bfloat16),
                            "state": torch.randn(N, HV, 128, 128, device=dev) * 0.1,
                        }
                        sets.append((inp, kda.alloc_outputs(w, dev)))
                    res = {}
                    for tile, pol, occ, g, sched in combos + [(0, 0, 0, 0, 0)]:
                        if tile and occ < 8 and N * HV * (128 // tile) <= 256 * occ:
                            continue  # the cap would not bind, or no unit would come from the queue
                        p = kda.params_for(w, tile_columns=tile, store_policy=pol, max_wg_per_cu=occ,
                                           column_groups=g, schedule=sched)
                        ws = kda.alloc_workspace(p, dev)
                        calls = [kda.PreparedVerify(p, a, o, ws) for a, o in sets]
                        for i in range(2 * nset):
                            calls[i % nset]()
                        reps = max(8, 2 * nset)
                        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                              for _ in range(reps)]
                        for i in range(reps):
                            ev[i][0].record()
                            calls[i % nset]()
                            ev[i][1].record()
                        torch.cuda.synchronize()
                        ms = sorted(a.elapsed_time(b) for a, b in ev)
                        key = f"{tile}/{pol}" + (f"/{occ}" if occ < 8 else "") + (f" g{g}" if g > 1 else "") + (
                            " q" if sched == 2 else "")
                        res[key if tile else "auto"] = ms[len(ms) // 2]
                    best = min((v, k) for k, v in res.items() if k != "auto")
                    auto_p = kda.params_for(w)
                    row = {"H": H, "HV": HV, "T": T, "N": N, "units": N * HV, "bytes": b_alg, "ms": res,
                           "best": best[1], "best_pct": 100 * b_alg / best[0] / 1e6 / HBM_PEAK_GBPS,
                           "auto_variant": kda.select_variant(auto_p),
                           "auto_over_best": res["auto"] / best[0]}
                    rows.append(row)
                    f.write(json.dumps(row) + "\n")
                    f.flush()
                    print(f"H={H:3d} HV={HV:3d} T={T} N={N:4d} units={N * HV:6d} best={best[1]:7s} "
                          f"{row['best_pct']:5.1f}% auto/best={row['auto_over_best']:.3f}", flush=True)
                    del sets
                    torch.cuda.empty_cache()
    worst = max(rows, key=lambda r: r["auto_over_best"])
    print(f"auto within {100 * (worst['auto_over_best'] - 1):.1f}% of the best combo on every shape "
          f"(worst: H={worst['H']} T={worst['T']} N={worst['N']})", flush=True)


def sweep_store(out_path: str) -> None:
    """Snapshot store policy sweep: on each shape, AUTO's launch (tile, cap, column groups,
    schedule) with the streaming stores (policy 1) and the device-scope streaming stores
    (policy 2), timed alternately. Shapes: T = 1..8, 256..32768 (sequence, value head)
    units, q/k heads shared by 1 or 2 value heads (H = 16, K = V = 128, bf16, softplus),
    buffers rotated so that >= 1 GiB is touched between reuses. One JSON object per shape."""
    import torch

    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    dev = torch.device("cuda:0")
    H = 16
    with open(out_path, "w") as f:
        for g in (1, 2):
            HV = H * g
            for T in range(1, 9):
                for units in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
                    N = units // HV
                    w = synth.Workload("sweep_store", N=N, T=T, H=H, HV=HV, K=128, V=128, dtype="bf16",
                                       gate="softplus", seed=1)
                    b_alg = synth.algorithmic_bytes(w)
                    nset = max(2, min(16, (1 << 30) // b_alg + 1))
                    sets = []
                    for _ in range(nset):
                        inp = {
                            "mixed_qkv": torch.randn(N, T, w.C, device=dev).to(torch.bfloat16),
                            "conv_weight": (torch.randn(w.C, 4, device=dev) * 0.5).to(torch.bfloat16),
                            "conv_state": torch.randn(N, w.C, 3, device=dev).to(torch.bfloat16),
                            "gate": torch.randn(N, T, HV, 128, device=dev).to(torch.bfloat16),
                            "A_log": torch.rand(HV, device=dev),
                            "dt_bias": torch.randn(HV * 128, device=dev) * 0.1,
                            "beta": torch.randn(N, T, HV, device=dev).to(torch.bfloat16),
                            "state": torch.randn(N, HV, 128, 128, device=dev) * 0.1,
                        }
                        sets.append((inp, kda.alloc_outputs(w, dev)))
                    launch = kda.select_launch(kda.params_for(w))
                    calls = {}
                    for pol in (1, 2):
                        p = kda.params_for(w, store_policy=pol)
                        ws = kda.alloc_workspace(p, dev)
                        calls[pol] = [kda.PreparedVerify(p, a, o, ws) for a, o in sets]
                    # one rotation over the buffer sets for both policies: consecutive calls never
                    # share a set, so neither policy reads what the other just left in the cache
                    for i in range(2 * nset):
                        for pol in (1, 2):
                            calls[pol][(2 * i + pol) % nset]()
                    reps = max(12, 2 * nset)
                    ev = {pol: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                for _ in range(reps)] for pol in (1, 2)}
                    for i in range(reps):
                        for pol in (1, 2):
                            ev[pol][i][0].record()
                            calls[pol][(2 * i + pol) % nset]()
                            ev[pol][i][1].record()
                    torch.cuda.synchronize()
                    ms = {pol: sorted(a.elapsed_time(b) for a, b in ev[pol])[reps // 2] for pol in (1, 2)}
                    pct = {pol: 100 * b_alg / ms[pol] / 1e6 / HBM_PEAK_GBPS for pol in (1, 2)}
                    row = {"H": H, "HV": HV, "T": T, "N": N, "units": units, "bytes": b_alg, "launch": launch,
                           "ms": ms, "pct": pct}
                    f.write(json.dumps(row) + "\n")
                    f.flush()
                    print(f"g={g} T={T} units={units:6d} auto_store={launch['store_policy']} "
                          f"nt {pct[1]:5.1f}%  nt+dev {pct[2]:5.1f}%", flush=True)
                    del sets, calls
                    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--device-warmup", type=float, default=0.3,
                    help="seconds of untimed calls before the warm-up steps (clock and power ramp)")
    ap.add_argument("--workload", default="large_batch")
    ap.add_argument("--variant", default="auto", choices=["auto", "small", "large"])
    ap.add_argument("--op", default="verify", choices=["verify", "verify_pooled", "commit", "unfused"],
                    help="verify (the headline), verify on pooled buffers with scattered rows, the accept "
                         "step, or the unfused two-kernel form of verify (same algorithmic bytes)")
    ap.add_argument("--tile", type=int, default=0, help="override: V columns per workgroup (32, 64, 128)")
    ap.add_argument("--store", type=int, default=0, help="override: snapshot stores, 1 streaming, 2 streaming at device scope")
    ap.add_argument("--occ", type=int, default=0, help="override: at most 1, 2, 4 or 6 workgroups per CU (8: no cap)")
    ap.add_argument("--groups", type=int, default=0, help="override: column groups of a whole-V workgroup (1, 2, 4)")
    ap.add_argument("--schedule", type=int, default=0,
                    help="override: 1 one workgroup per unit, 2 resident workgroups pulling units from a queue")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--sweep", default=None, metavar="OUT.jsonl",
                    help="run the H x T x N sweep over tile widths and store policies instead")
    ap.add_argument("--sweep-quick", action="store_true", help="a reduced sweep grid")
    ap.add_argument("--sweep-store", default=None, metavar="OUT.jsonl",
                    help="time AUTO's launch with store policy 1 and 2 over T x units x shared heads")
    ap.add_argument("--sweep-h", default="", help="comma-separated H values for --sweep (default all)")
    ap.add_argument("--sweep-g", type=int, default=1, help="value heads per q/k head for --sweep (HV = g H)")
    ap.add_argument("--sweep-t", default="", help="comma-separated T values for --sweep (default 1,2,4,6,8)")
    ap.add_argument("--sweep-units", default="", metavar="LO,HI",
                    help="keep only the --sweep shapes with LO <= N HV <= HI units")
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

    if args.sweep:
        sweep(args.sweep, args.sweep_quick, [int(x) for x in args.sweep_h.split(",") if x], args.sweep_g,
              [int(x) for x in args.sweep_t.split(",") if x],
              tuple(int(x) for x in args.sweep_units.split(",")) if args.sweep_units else None)
        return
    if args.sweep_store:
        sweep_store(args.sweep_store)
        return

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
    p = kda.params_for(w, variant=variant, tile_columns=args.tile, store_policy=args.store,
                       max_wg_per_cu=args.occ, column_groups=args.groups, schedule=args.schedule)
    resolved = {kda.VARIANT_SMALL: "small", kda.VARIANT_LARGE: "large"}[kda.select_variant(p)]
    print(f"[bench] workload={w.name} N={w.N} T={w.T} H={w.H} HV={w.HV} K={w.K} V={w.V} "
          f"{w.dtype} {w.gate} variant={resolved}", file=sys.stderr, flush=True)
    inp_cpu = synth.make_inputs(w)
    inp = {k: v.to(dev) for k, v in inp_cpu.items()}
    out = kda.alloc_outputs(w, dev)
    ws = kda.alloc_workspace(p, dev)
    stream = torch.cuda.current_stream()

    nset = 1
    if args.op == "verify":
        # Rotate distinct buffer sets so that >= 1 GiB is touched between reuses: a workload
        # smaller than that would otherwise run partly from the 256 MB last-level cache.
        b_alg = synth.algorithmic_bytes(w)
        nset = max(1, min(8, -(-(1 << 30) // b_alg)))
        sets = [(inp, out)] + [({k: v.clone() for k, v in inp.items()}, kda.alloc_outputs(w, dev))
                               for _ in range(nset - 1)]
        calls = [kda.PreparedVerify(p, a, o, ws, stream) for a, o in sets]  # checks once; one C call each
        rot = [0]

        def step():
            calls[rot[0] % nset]()
            rot[0] += 1
    elif args.op == "unfused":
        act = torch.empty((w.N, w.T, w.C), dtype=torch.float32, device=dev)
        b_alg = synth.algorithmic_bytes(w)  # the fused step's bytes, so the fractions compare directly
        nset = max(1, min(8, -(-(1 << 30) // b_alg)))  # rotated like the fused step
        sets = [(inp, out)] + [({k: v.clone() for k, v in inp.items()}, kda.alloc_outputs(w, dev))
                               for _ in range(nset - 1)]
        rot = [0]

        def step():
            a, o = sets[rot[0] % nset]
            rot[0] += 1
            kda.kda_conv_verify_decode_unfused(p, None, a["mixed_qkv"], a["conv_weight"], a["conv_state"],
                                               a["gate"], a["A_log"], a["dt_bias"], a["beta"], a["state"],
                                               o["o"], o["inter_ssm"], o["conv_window"], act, ws, stream)
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

    # The part ramps its clocks over the first tens of milliseconds of sustained work: run
    # untimed calls for --device-warmup seconds first (reported as device_warmup_calls).
    dw_calls = 0
    t_end = time.perf_counter() + args.device_warmup
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        dw_calls += 10
        torch.cuda.synchronize()
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

    launch = kda.select_launch(p)
    traffic = measured_traffic(w.name, resolved, launch) if args.op == "verify" else None
    copy_gbps = device_copy_gbps(b_alg, dev) if args.op == "verify" else None
    cpu = None
    if not args.no_cpu_baseline and args.op == "verify":
        print("[bench] timing the float64 oracle on a bounded sample (cpu_baseline)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp_cpu, args.cpu_budget, host_threads())

    line = {
        "metric": "verify tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": tokens / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "device_warmup_calls": dw_calls,
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
            "in_dtype": w.dtype, "state_dtype": "f32", "gate": w.gate, "variant": resolved, "launch": launch,
            "algorithmic_bytes_per_call": b_alg, "buffer_sets": nset,
            "hbm_gbps": achieved, "pct_of_hbm_peak": 100 * achieved / HBM_PEAK_GBPS,
            "device_copy_gbps": copy_gbps,
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
