"""Benchmark of the fused causal-conv1d + KDA multi-token verify step on one MI355X.

One step = one fused verify call (conv + SiLU, l2norm, gate, beta, gated delta rule
over T tokens, snapshots, conv window and rolled cache) over the whole batch, with
inputs already resident in HBM. Prints one JSON line:

  value      verify tokens/s = N*T / (time per call)
  roofline   algorithmic HBM bytes per call / average kernel duration (HIP events on
             the launch stream), against the MI355X HBM peak of 8 TB/s
  cpu_baseline  the float64 oracle on bounded samples of the same workload, on all host
                threads (sequence slices) and on one thread; its `parity` compares one
                fresh GPU call on the same inputs with the oracle on the multi-thread
                sample (max |error| of o and inter_ssm against 2e-3, conv window and
                rolled cache bit for bit)

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
PARITY_TOL = 2e-3  # max |error| of o and inter_ssm the GPU parity tests accept


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


def cpu_baseline(w, inp_cpu, budget_s: float, threads: int, gpu_out=None):
    """The oracle as it is (float64, sequential C) on bounded samples of the same inputs,
    run on slices of 4 sequences: (1) on one host thread over the first n sequences, n
    chosen from a one-slice probe to take about budget_s / 2; (2) on all `threads` host
    threads, each running the oracle on its own slices (ctypes releases the GIL), over as
    many of the batch's sequences as fit in about budget_s / 2 (short samples repeated).
    With `gpu_out` (the device outputs of one call on these inputs, conv_state rolled in
    place), one more untimed pass over sample (2) compares them with the oracle."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

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

    parity = None
    if gpu_out is not None:
        import torch

        def same_bits(got, ref64):
            ref = torch.from_numpy(ref64).to(got.dtype)
            iview = torch.int16 if got.element_size() == 2 else torch.int32
            return bool(torch.equal(got.view(iview), ref.view(iview)))

        def compare_slice(ab):
            a, b = ab
            part = {k: (v[a:b].contiguous() if k in per_seq else v) for k, v in inp_cpu.items()}
            ref = oracle.verify_workload(w.with_(N=b - a), part)
            e_o = float(np.abs(gpu_out["o"][a:b].double().cpu().numpy() - ref["o"]).max())
            e_s = float(np.abs(gpu_out["inter_ssm"][a:b].cpu().numpy() - ref["inter_ssm"]).max())
            return (e_o, e_s, same_bits(gpu_out["conv_window"][a:b].cpu(), ref["conv_window"]),
                    same_bits(gpu_out["conv_state"][a:b].cpu(), ref["conv_state"]))

        with ThreadPoolExecutor(threads) as ex:
            res = list(ex.map(compare_slice, slices(n_mt)))
        e_o = max(r[0] for r in res)
        e_s = max(r[1] for r in res)
        parity = {
            "sequences": n_mt,
            "o_max_abs_err": e_o,
            "inter_ssm_max_abs_err": e_s,
            "tolerance": PARITY_TOL,
            "conv_window_bit_exact": all(r[2] for r in res),
            "conv_state_bit_exact": all(r[3] for r in res),
        }
        parity["pass"] = bool(e_o <= PARITY_TOL and e_s <= PARITY_TOL and parity["conv_window_bit_exact"]
                              and parity["conv_state_bit_exact"])
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
        "parity": parity,
    }


def sweep_launches() -> dict:
    """The launches the dispatch sweep times on every shape (K = V = 128), by name: the
    32-column split; whole-V grids without a cap in 1, 2 or 4 column groups, each unit
    order (o1 XCD ranges, o2 pairs) and store policy (s1 streaming, s2 streaming at device
    scope); capped grids (one or two workgroups per CU; 64 columns at two per CU); the queue
    at one workgroup per CU in 1, 2 or 4 column groups; and the stream with the next state
    tile loaded after the conv (p1) or at the start (p2)."""
    L = {"split32 s1": dict(tile_columns=32, max_wg_per_cu=8, store_policy=1, unit_order=1)}
    for g in (1, 2, 4):
        for st in (1, 2):
            for o in (1, 2):
                L[f"grid g{g} s{st} o{o}"] = dict(tile_columns=128, max_wg_per_cu=8, column_groups=g,
                                                  store_policy=st, unit_order=o)
    for g in (1, 2):
        for st in (1, 2):
            L[f"cap1 g{g} s{st}"] = dict(tile_columns=128, max_wg_per_cu=1, column_groups=g, store_policy=st,
                                         unit_order=1)
    for st in (1, 2):
        L[f"cap2 g1 s{st}"] = dict(tile_columns=128, max_wg_per_cu=2, store_policy=st, unit_order=1)
        L[f"cap2 64c s{st}"] = dict(tile_columns=64, max_wg_per_cu=2, store_policy=st, unit_order=1)
    for g in (1, 2, 4):
        for st in (1, 2):
            L[f"queue g{g} s{st}"] = dict(tile_columns=128, max_wg_per_cu=1, column_groups=g, store_policy=st,
                                          schedule=2)
    for pf in (1, 2):
        L[f"stream s2 p{pf}"] = dict(tile_columns=128, store_policy=2, schedule=3, prefetch=pf)
    return L


def launch_name(ln: dict) -> str:
    """The sweep's name for a launch reported by select_launch."""
    if ln["schedule"] == 3:
        return f"stream s{ln['store_policy']} p{ln['prefetch']}"
    if ln["schedule"] == 2:
        return f"queue g{ln['column_groups']} s{ln['store_policy']}"
    if ln["tile_columns"] == 32:
        return f"split32 s{ln['store_policy']}"
    if ln["max_wg_per_cu"]:
        if ln["tile_columns"] == 64:
            return f"cap{ln['max_wg_per_cu']} 64c s{ln['store_policy']}"
        return f"cap{ln['max_wg_per_cu']} g{ln['column_groups']} s{ln['store_policy']}"
    if ln["tile_columns"] == 64:
        return f"grid 64c s{ln['store_policy']}"
    return f"grid g{ln['column_groups']} s{ln['store_policy']} o{ln['unit_order']}"


def sweep(out_path: str, hs, gs, ts, ns, units_range, rounds: int = 2) -> None:
    """Dispatch sweep (K = V = 128, bf16, softplus gate): on every shape H x (HV = g H) x T x
    N with units = N HV inside units_range, each launch of sweep_launches() and AUTO's own
    launch, round-robin over `rounds` rounds. In each round a launch gets one untimed pass
    over the shape's buffer sets and then a median over >= 8 timed calls (HIP events); the
    buffer sets rotate so that >= 1 GiB is touched between reuses of a set. A cap is timed
    only where it binds (more workgroups than cap x 256 CUs), the queue and the stream only
    from 512 units (the stream up to T = 8),
    the 32-column split only up to 512 units. One JSON object per shape: the mean over the
    rounds of each launch's median time, and AUTO's launch."""
    import torch

    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    dev = torch.device("cuda:0")
    launches = sweep_launches()
    with open(out_path, "w") as f:
        for g in gs:
            for H in hs:
                HV = g * H
                for T in ts:
                    for N in ns:
                        units = N * HV
                        if not units_range[0] <= units <= units_range[1]:
                            continue
                        w = synth.Workload("sweep", N=N, T=T, H=H, HV=HV, K=128, V=128, dtype="bf16",
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
                        todo = {}
                        for name, kw in list(launches.items()) + [("auto", {})]:
                            cap = kw.get("max_wg_per_cu", 8)
                            wgs = units * (128 // kw.get("tile_columns", 128))
                            if kw.get("schedule", 0) >= 2 and units < 512:
                                continue
                            if kw.get("schedule") == 3 and T > 8:
                                continue
                            if kw.get("schedule", 0) < 2 and cap < 8 and wgs <= 256 * cap:
                                continue
                            if kw.get("tile_columns") == 32 and units > 512:
                                continue
                            p = kda.params_for(w, **kw)
                            ws = kda.alloc_workspace(p, dev)
                            todo[name] = [kda.PreparedVerify(p, a, o, ws) for a, o in sets]
                        times = {k: [] for k in todo}
                        reps = max(8, nset)
                        for _ in range(rounds):
                            for name, calls in todo.items():
                                for i in range(nset):
                                    calls[i]()
                                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                      for _ in range(reps)]
                                for i in range(reps):
                                    ev[i][0].record()
                                    calls[i % nset]()
                                    ev[i][1].record()
                                torch.cuda.synchronize()
                                ms = sorted(a.elapsed_time(b) for a, b in ev)
                                times[name].append(ms[len(ms) // 2])
                        res = {k: sum(v) / len(v) for k, v in times.items()}
                        auto = kda.select_launch(kda.params_for(w))
                        best = min((v, k) for k, v in res.items() if k != "auto")
                        row = {"H": H, "HV": HV, "T": T, "N": N, "units": units, "bytes": b_alg, "ms": res,
                               "auto": auto, "auto_name": launch_name(auto), "best": best[1],
                               "auto_over_best": res["auto"] / best[0]}
                        f.write(json.dumps(row) + "\n")
                        f.flush()
                        print(f"H={H:3d} HV={HV:3d} T={T} N={N:4d} units={units:6d} best={best[1]:16s} "
                              f"{100 * b_alg / best[0] / 1e6 / HBM_PEAK_GBPS:5.1f}% auto={row['auto_name']:16s} "
                              f"auto/best={row['auto_over_best']:.3f}", flush=True)
                        del sets, todo
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
    ap.add_argument("--op", default="verify",
                    choices=["verify", "verify_pooled", "commit", "unfused", "serve", "serve_no_commit"],
                    help="verify (the headline), verify on pooled buffers with scattered rows, the accept "
                         "step, or the unfused two-kernel form of verify (same algorithmic bytes)")
    ap.add_argument("--tile", type=int, default=0, help="override: V columns per workgroup (32, 64, 128)")
    ap.add_argument("--store", type=int, default=0, help="override: snapshot stores, 1 streaming, 2 streaming at device scope")
    ap.add_argument("--occ", type=int, default=0, help="override: at most 1, 2, 4 or 6 workgroups per CU (8: no cap)")
    ap.add_argument("--groups", type=int, default=0, help="override: column groups of a whole-V workgroup (1, 2, 4)")
    ap.add_argument("--schedule", type=int, default=0,
                    help="override: 1 one workgroup per unit, 2 resident workgroups pulling units from a queue, "
                         "3 the queue with a producer wave loading the next unit into LDS")
    ap.add_argument("--prefetch", type=int, default=0,
                    help="override (schedule 3): load the next state tile 1 after the conv, 2 at the start")
    ap.add_argument("--order", type=int, default=0,
                    help="override: unit order of the grid, 1 XCD ranges, 2 pairs of units dealt to the XCDs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--sweep", default=None, metavar="OUT.jsonl",
                    help="run the dispatch sweep (every launch of sweep_launches() and AUTO's on each shape) "
                         "instead of the benchmark")
    ap.add_argument("--sweep-h", default="8,16,32,64", help="comma-separated H values for --sweep")
    ap.add_argument("--sweep-g", default="1,2", help="comma-separated value heads per q/k head for --sweep")
    ap.add_argument("--sweep-t", default="1,2,3,4,6,8", help="comma-separated T values for --sweep")
    ap.add_argument("--sweep-n", default="2,4,6,8,12,16,24,32,48,64,96,128,192,256",
                    help="comma-separated N values for --sweep")
    ap.add_argument("--sweep-units", default="128,4096", metavar="LO,HI",
                    help="keep only the --sweep shapes with LO <= N HV <= HI units")
    ap.add_argument("--sweep-rounds", type=int, default=2, help="round-robin rounds per shape for --sweep")
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
        ints = lambda x: [int(v) for v in x.split(",") if v]  # noqa: E731
        sweep(args.sweep, ints(args.sweep_h), ints(args.sweep_g), ints(args.sweep_t), ints(args.sweep_n),
              tuple(ints(args.sweep_units)), args.sweep_rounds)
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
                       max_wg_per_cu=args.occ, column_groups=args.groups, schedule=args.schedule,
                       unit_order=args.order, prefetch=args.prefetch)
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
    elif args.op in ("serve", "serve_no_commit"):
        # One serving step of a batch whose sequences all advance, sequence n accepting
        # n % T + 1 tokens: with the accept step (verify on a state and a conv-cache pool,
        # then commit into them), or without it (the verify reads each sequence's accepted
        # snapshot row of the previous step's inter_ssm and conv_window, viewed as N*T state
        # and conv-cache rows, and writes its own to a second set; the two sets alternate).
        acc = (torch.arange(w.N, dtype=torch.int32) % w.T + 1).to(dev)
        s_in = 2 if w.dtype == "bf16" else 4
        if args.op == "serve":
            ident = kda.make_pools(w.N)

            def step():
                kda.kda_conv_verify_decode_pooled(p, ident, inp["mixed_qkv"], inp["conv_weight"], inp["conv_state"],
                                                  inp["gate"], inp["A_log"], inp["dt_bias"], inp["beta"], inp["state"],
                                                  out["o"], out["inter_ssm"], out["conv_window"], ws, stream)
                kda.verify_commit(p, ident, acc, out["inter_ssm"], out["conv_window"], inp["state"], inp["conv_state"],
                                  stream)
            b_alg = (synth.algorithmic_bytes(w) + w.N * (2 * 4 * w.HV * w.K * w.V + 2 * 3 * s_in * w.C)
                     + 4 * 4 * w.N)
        else:
            NT = w.N * w.T
            rows = torch.arange(w.N, dtype=torch.int32, device=dev) * w.T + acc - 1
            snap_pools = kda.make_pools(w.N, rows, rows, None, NT, NT, w.N)
            bufs = [out, kda.alloc_outputs(w, dev)]
            kda.run(p, inp, bufs[1], ws)  # a first step from the inputs fills one set
            par = [1]

            def step():
                prev, cur = bufs[par[0]], bufs[1 - par[0]]
                par[0] = 1 - par[0]
                kda.kda_conv_verify_decode_pooled(p, snap_pools, inp["mixed_qkv"], inp["conv_weight"],
                                                  prev["conv_window"].view(NT, w.C, 3), inp["gate"], inp["A_log"],
                                                  inp["dt_bias"], inp["beta"],
                                                  prev["inter_ssm"].view(NT, w.HV, w.K, w.V), cur["o"],
                                                  cur["inter_ssm"], cur["conv_window"], ws, stream)
            b_alg = synth.algorithmic_bytes(w) + 2 * 4 * w.N
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
        # one more call on a pristine copy of the inputs, for the parity readout
        fresh = {k: v.to(dev) for k, v in inp_cpu.items()}
        fresh_out = kda.alloc_outputs(w, dev)
        kda.run(p, fresh, fresh_out, ws, stream)
        torch.cuda.synchronize()
        fresh_out["conv_state"] = fresh["conv_state"]
        print("[bench] timing the float64 oracle on a bounded sample (cpu_baseline)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp_cpu, args.cpu_budget, host_threads(), fresh_out)
        del fresh, fresh_out
        par = cpu["parity"]
        print(f"[bench] parity on {par['sequences']} sequences: o {par['o_max_abs_err']:.2e}, inter_ssm "
              f"{par['inter_ssm_max_abs_err']:.2e} (tolerance {PARITY_TOL}), conv window bits "
              f"{par['conv_window_bit_exact']}, conv cache bits {par['conv_state_bit_exact']}", file=sys.stderr,
              flush=True)

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
