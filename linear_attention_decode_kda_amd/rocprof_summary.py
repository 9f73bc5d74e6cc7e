"""Summarise rocprofv3 CSV output of the verify kernel into short text for profiles/.

  python -m linear_attention_decode_kda_amd.rocprof_summary stats <kernel_stats.csv> <cmd> <out.md>
  python -m linear_attention_decode_kda_amd.rocprof_summary traffic <workload> <variant>
         <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> <cmd-file> <out.json>

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
KERNEL_TAG = "kda_verify_kernel"


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


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:5])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    else:
        raise SystemExit(__doc__)
