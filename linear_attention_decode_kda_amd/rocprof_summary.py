"""Summarise rocprofv3 CSV output of the verify kernel into short text for profiles/.

  python -m linear_attention_decode_kda_amd.rocprof_summary stats <kernel_stats.csv> <cmd> <out.md>
  python -m linear_attention_decode_kda_amd.rocprof_summary traffic <workload> <variant>
         <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> <cmd-file> <out.json>
  python -m linear_attention_decode_kda_amd.rocprof_summary sweep-md <sweep.jsonl> <cmd> <out.md> [refs]
  python -m linear_attention_decode_kda_amd.rocprof_summary store-md <sweep_store.jsonl> <cmd> <out.md>

`traffic` scales the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of the verify
kernel by what the same counters read for a plain 1 GiB device copy (read 1 GiB, write
1 GiB), and records the hash of the kernel source the counters were taken on, so that a
later kernel change makes the figure stale (bench.py then reports traffic as null).
"""
from __future__ import annotations

import csv
import json
import os
import statistics
import sys

COPY_BYTES = 1 << 30
KERNEL_TAG = "kda::kda_verify"  # the grid kernel (kda_verify_kernel) and the queue kernel


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _counter(path, name, tag):
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if r.get("Counter_Name") == name and tag in r.get("Kernel_Name", "")]
    if not vals:
        raise SystemExit(f"no {name} rows for {tag!r} in {path}")
    return statistics.median(vals), len(vals)


def stats(csv_path: str, cmd: str, out: str) -> None:
    rows = _rows(csv_path)
    lines = [f"# rocprofv3 kernel statistics", "", f"Command: `{cmd}`", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def store_md(jsonl: str, cmd: str, out: str) -> None:
    """Table of the store-policy sweep (bench.py --sweep-store) with the policy the library's
    AUTO rule picks for each shape now (host-only call, no GPU)."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import linear_attention_decode_kda_amd as kda

    rows = [json.loads(l) for l in open(jsonl) if l.strip()]
    lines = ["# Snapshot store policy sweep (K = V = 128, bf16, softplus gate, H = 16)", "",
             f"Command: `{cmd}`", "",
             "AUTO's launch (tile, cap, column groups, schedule) timed with the streaming stores (1: `nt`) and "
             "the streaming stores at device scope (2: `nt sc1`), alternately over distinct buffer sets (>= 1 GiB "
             "touched between reuses of a set); median of >= 12 calls each. Percent of the 8 TB/s HBM peak = "
             "algorithmic bytes / kernel time. `AUTO` is the policy the library picks for the shape.", "",
             "| value heads per q/k head | T | units | 1: nt % | 2: nt sc1 % | AUTO |", "|---|---|---|---|---|---|"]
    gain = []
    for r in rows:
        g = r["HV"] // r["H"]
        p = kda.make_params(r["N"], r["T"], r["H"], r["HV"], 128, 128)
        auto = kda.select_launch(p)["store_policy"]
        p1, p2 = r["pct"]["1"], r["pct"]["2"]
        gain.append((max(p1, p2) - (p1 if auto == 1 else p2)))
        lines.append(f"| {g} | {r['T']} | {r['units']} | {p1:.1f} | {p2:.1f} | {auto} |")
    lines += ["", f"AUTO's pick is within {max(gain):.1f} points of the faster policy on every shape "
              f"(mean {statistics.mean(gain):.2f} points)."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic(workload, variant, fetch, write, cfetch, cwrite, cmd_file, out) -> None:
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import source_hash  # the same hash bench.py checks
    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    kf, nf = _counter(fetch, "FETCH_SIZE", KERNEL_TAG)
    kw, nw = _counter(write, "WRITE_SIZE", KERNEL_TAG)
    cf, _ = _counter(cfetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter(cwrite, "WRITE_SIZE", "copyBuffer")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    read_b = kf * 1024.0 * f_scale
    write_b = kw * 1024.0 * w_scale
    alg = synth.algorithmic_bytes(synth.WORKLOADS[workload])
    with open(cmd_file) as f:
        cmds = [ln.strip() for ln in f if ln.strip()]
    doc = {
        "workload": workload,
        "variant": variant,
        "launch": kda.select_launch(kda.params_for(synth.WORKLOADS[workload])),
        "source_hash": source_hash(),
        "commands": cmds,
        "kernel_fetch_kib_per_dispatch": kf,
        "kernel_write_kib_per_dispatch": kw,
        "dispatches": [nf, nw],
        "copy_1gib_fetch_kib": cf,
        "copy_1gib_write_kib": cw,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_read_bytes_per_call": read_b,
        "hbm_write_bytes_per_call": write_b,
        "hbm_bytes_per_call": read_b + write_b,
        "algorithmic_bytes_per_call": alg,
        "traffic_over_algorithmic": (read_b + write_b) / alg,
    }
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def sweep_md(jsonl: str, cmd: str, out: str, refs: str = "") -> None:
    """Table of a `bench.py --sweep` run: per shape the best (tile/store[/cap]) and its
    share of the HBM peak, the AUTO choice and its share, and reference launches (refs,
    comma-separated combination labels; four by default)."""
    import linear_attention_decode_kda_amd as kda

    rows = [json.loads(ln) for ln in open(jsonl) if ln.strip()]
    pct = lambda r, k: 100.0 * r["bytes"] / r["ms"][k] / 1e6 / 8000.0 if k in r["ms"] else float("nan")
    refs = tuple(refs.split(",")) if refs else ("32/1", "128/1", "128/1/1", "128/1/1 q")
    g = rows[0].get("HV", rows[0]["H"]) // rows[0]["H"]
    title = "H = HV" if g == 1 else f"H, HV = {g} H"
    lines = [f"# {title} x T x N sweep of the verify kernel (K = V = 128, bf16, softplus gate)", "",
             f"Command: `{cmd}` (one MI355X; each shape's buffers rotated so that >= 1 GiB is touched "
             "between reuses; median of >= 8 calls per combination), summarised by "
             f"`python -m linear_attention_decode_kda_amd.rocprof_summary sweep-md {os.path.basename(jsonl)} ...`.",
             "",
             "Combinations are tile/store[/cap][ gN][ q]: V columns per workgroup, snapshot store policy "
             "(1 streaming, 2 the library's policy 2 at the time of the run), the workgroups-per-CU cap (none, 6, 4, 2, 1; a cap is timed "
             "only where the grid has more workgroups than it lets run at once), column groups of a "
             "whole-V workgroup (gN), and q for the queue schedule (resident workgroups pulling units; "
             "otherwise one workgroup per unit). Percent of the 8 TB/s HBM "
             "peak = algorithmic bytes / kernel time. Shapes of <= 128 units are launch-latency-bound: "
             "their timings include the launch, and the columns differ by noise.", "",
             "| H | HV | T | N | units | best | best % | AUTO | AUTO % | AUTO/best | " + " | ".join(refs) + " |",
             "|---|---|---|---|---|---|---|---|---|---|" + "---|" * len(refs)]
    for r in rows:
        p = kda.make_params(r["N"], r["T"], r["H"], r.get("HV", r["H"]), 128, 128)
        ln = kda.select_launch(p)
        auto = (f"{ln['tile_columns']}/{ln['store_policy']}" + (f"/{ln['max_wg_per_cu']}" if ln["max_wg_per_cu"] else "")
                + (f" g{ln['column_groups']}" if ln["column_groups"] > 1 else "")
                + (" q" if ln.get("schedule") == 2 else ""))
        lines.append(f"| {r['H']} | {r.get('HV', r['H'])} | {r['T']} | {r['N']} | {r['units']} | {r['best']} | "
                     f"{r['best_pct']:.1f} | {auto} | "
                     f"{pct(r, 'auto'):.1f} | {r['auto_over_best']:.3f} | "
                     + " | ".join(f"{pct(r, k):.1f}" if k in r["ms"] else "-" for k in refs) + " |")
    mean = statistics.mean(r["auto_over_best"] for r in rows)
    big = [r for r in rows if r["units"] >= 256]
    lines += ["", f"AUTO over best, mean over all {len(rows)} shapes: {mean:.3f}; over the {len(big)} shapes "
              f"of >= 256 units: {statistics.mean(r['auto_over_best'] for r in big):.3f}."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    elif sys.argv[1] == "sweep-md":
        sweep_md(*sys.argv[2:6])
    elif sys.argv[1] == "store-md":
        store_md(*sys.argv[2:5])
    else:
        raise SystemExit(__doc__)
