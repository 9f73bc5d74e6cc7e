"""Summarise rocprofv3 CSV output of the verify kernel into short text for profiles/.

  python -m linear_attention_decode_kda_amd.rocprof_summary stats <kernel_stats.csv> <cmd> <out.md>
  python -m linear_attention_decode_kda_amd.rocprof_summary traffic <workload> <variant>
         <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> <cmd-file> <out.json>
  python -m linear_attention_decode_kda_amd.rocprof_summary sweep-md <sweep.jsonl> <cmd> <out.md>

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


def _bucket(units: int) -> str:
    return ("<= 128" if units <= 128 else "129-512" if units <= 512 else "513-1023" if units < 1024
            else "1024-2047" if units < 2048 else ">= 2048")


def sweep_md(jsonl: str, cmd: str, out: str) -> None:
    """Table of a `bench.py --sweep` run (the dispatch sweep): per shape the fastest launch
    and its share of the HBM peak, the launch AUTO ran at the time of the sweep, and the
    launch the library's rule picks now (host-only call) with its time over the fastest."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    import linear_attention_decode_kda_amd as kda

    rows = [json.loads(ln) for ln in open(jsonl) if ln.strip()]
    pct = lambda r, ms: 100.0 * r["bytes"] / ms / 1e6 / 8000.0  # noqa: E731
    lines = [f"# Dispatch sweep of the verify kernel (K = V = 128, bf16, softplus gate)", "",
             f"Command: `{cmd}` (one MI355X), summarised by "
             f"`python -m linear_attention_decode_kda_amd.rocprof_summary sweep-md {os.path.basename(jsonl)} ...`.",
             "",
             "Every shape's launches were timed round-robin (each: an untimed pass over the buffer sets, then the "
             "median of >= 8 calls from HIP events, in each of two rounds; the mean of the rounds), over buffer "
             "sets rotated so that >= 1 GiB is touched between reuses of a set. Launch names: `split32` the "
             "32-column split; `grid gG` whole-V workgroups without a cap in G column groups; `capC` at most C "
             "workgroups per CU (`64c`: 64 columns); `queue gG` one resident workgroup per CU pulling units; "
             "`stream pP` the queue with a producer wave loading the next unit into LDS, its state tile after the "
             "conv (p1) or at the start (p2); "
             "`s1` streaming stores, `s2` streaming at device scope; `o1` XCD-range unit order, `o2` pairs. "
             "Percent of the 8 TB/s HBM peak = algorithmic bytes / time (launch gap included). `rule` is the "
             "launch the library picks now; `rule/best` its time over the fastest launch (nan where this sweep did "
             "not time that launch).", "",
             "| H | HV | T | N | units | fastest | % | AUTO at the time | rule now | rule % | rule/best |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    regs, per = [], {}
    for r in rows:
        best_ms = min(v for k, v in r["ms"].items() if k != "auto")
        ln = kda.select_launch(kda.make_params(r["N"], r["T"], r["H"], r["HV"], 128, 128))
        name = bench.launch_name(ln)
        ms = r["ms"].get(name)
        if ms is None and name == r.get("auto_name"):
            ms = r["ms"].get("auto")
        reg = ms / best_ms if ms else float("nan")
        if ms:
            regs.append(reg)
            per.setdefault(_bucket(r["units"]), []).append(reg)
        lines.append(f"| {r['H']} | {r['HV']} | {r['T']} | {r['N']} | {r['units']} | {r['best']} | "
                     f"{pct(r, best_ms):.1f} | {r.get('auto_name', '-')} | {name} | "
                     f"{pct(r, ms) if ms else float('nan'):.1f} | {reg:.3f} |")
    lines += ["", f"Rule now over the fastest launch, over the {len(regs)} shapes whose rule launch was timed: mean "
              f"{statistics.mean(regs):.3f}, worst {max(regs):.3f}.", "",
              "| units | shapes | mean rule/best |", "|---|---|---|"]
    for b in ("<= 128", "129-512", "513-1023", "1024-2047", ">= 2048"):
        if b in per:
            lines.append(f"| {b} | {len(per[b])} | {statistics.mean(per[b]):.3f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    elif sys.argv[1] == "sweep-md":
        sweep_md(*sys.argv[2:5])
    else:
        raise SystemExit(__doc__)
