"""Per-phase timeline of the verify kernel: a profiling tool, not part of the library.

`build` writes an instrumented copy of csrc/kda_verify.hip into _build/timeline/ and compiles
it (CPU only, hipcc cross-compiles): thread 0 of every workgroup reads the 100 MHz real-time
counter (s_memrealtime) at each phase boundary of a unit (entry, staged inputs visible,
conv + gate done, l2norm done, every token's reduction barrier and snapshot stores, end of
the unit, its stores drained) and writes the sixteen stamps, with its XCD id, into a buffer
the host passes in. The copy is otherwise the library's kernel source, so the launch
configuration and the arithmetic are the library's (the stamps and the drain wait at the
end of each unit add a little time).

`run` loads that copy in place of the library (in this process only), runs the AUTO launch
of each named workload with stamps on, and prints a markdown table: call span, median phase
durations, and per-XCD end times and unit durations.

  python -m linear_attention_decode_kda_amd.timeline build
  python -m linear_attention_decode_kda_amd.timeline run small_batch gva large_batch > out.md
  python -m linear_attention_decode_kda_amd.timeline run gva gva:schedule=2,max_wg_per_cu=1,tile_columns=128
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
OUT = os.path.join(ROOT, "_build", "timeline")
SRC = os.path.join(OUT, "kda_timeline.hip")
LIB = os.path.join(OUT, "libkda_timeline.so")

NAMES = ["entry", "staged inputs", "conv + gate", "barrier", "l2norm"] + \
    sum([[f"token {t} reduction", f"token {t} update + stores"] for t in range(4)], []) + ["tail", "drain"]


def _instrument(src: str) -> str:
    def sub(old, new):
        nonlocal src
        if src.count(old) != 1:
            raise SystemExit(f"timeline: kernel source changed, cannot place a stamp at: {old[:60]!r}")
        src = src.replace(old, new)

    now = "__builtin_amdgcn_s_memrealtime()"
    sub("  int gate_mode;\n", "  int gate_mode;\n  unsigned long long* stamps;\n")
    sub("  const int tid = threadIdx.x;\n  // The ticket",
        f"  const int tid = threadIdx.x;\n  unsigned long long st_[16];\n  st_[0] = {now};\n  // The ticket")
    sub("  __syncthreads();  // B0:", f"  __syncthreads();  st_[1] = {now};  // B0:")
    sub("  __syncthreads();  // B1\n", f"  st_[2] = {now};\n  __syncthreads();  // B1\n  st_[3] = {now};\n")
    sub("  __syncthreads();  // B2\n", f"  __syncthreads();  // B2\n  st_[4] = {now};\n")
    sub("    __syncthreads();\n    const int w0 = grp * CF::NW;",
        "    __syncthreads();\n    { const unsigned long long n_ = " + now + "; if (t == 0) st_[5] = n_; "
        "else if (t == 1) st_[7] = n_; else if (t == 2) st_[9] = n_; else if (t == 3) st_[11] = n_; }\n"
        "    const int w0 = grp * CF::NW;")
    sub("      store_snapshot<CF::STP>(dst + (size_t)r * Q * V, sv);\n    }\n",
        "      store_snapshot<CF::STP>(dst + (size_t)r * Q * V, sv);\n    }\n"
        "    { const unsigned long long n_ = " + now + "; if (t == 0) st_[6] = n_; "
        "else if (t == 1) st_[8] = n_; else if (t == 2) st_[10] = n_; else if (t == 3) st_[12] = n_; }\n")
    marker = "// Grid schedule: one workgroup per unit;"
    end = src.rindex("\n}\n", 0, src.index(marker))  # the closing brace of verify_unit
    src = src[:end] + f"""
  st_[13] = {now};
  __builtin_amdgcn_s_waitcnt(0);
  st_[14] = {now};
  if (tid == 0 && a.stamps) {{
    unsigned int xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    st_[15] = xcc;
    for (int q = 0; q < 16; ++q) a.stamps[(size_t)lb * 16 + q] = st_[q];
  }}
""" + src[end:]
    sub("  a.gate_mode = p->gate_mode;\n", "  a.gate_mode = p->gate_mode;\n  a.stamps = g_stamps;\n")
    sub("kda_status launch_verify(const kda_verify_params* p, const PoolView& pv, const void* mixed_qkv,\n"
        "                         const void* conv_weight, void* conv_state, const void* gate, const float* A_log,\n"
        "                         const float* dt_bias, const void* beta, const float* state, void* o, float* inter_ssm,\n"
        "                         void* conv_window, void* workspace, hipStream_t stream, bool pre) {",
        "unsigned long long* g_stamps = nullptr;\n"
        "kda_status launch_verify(const kda_verify_params* p, const PoolView& pv, const void* mixed_qkv,\n"
        "                         const void* conv_weight, void* conv_state, const void* gate, const float* A_log,\n"
        "                         const float* dt_bias, const void* beta, const float* state, void* o, float* inter_ssm,\n"
        "                         void* conv_window, void* workspace, hipStream_t stream, bool pre) {")
    src += '\nextern "C" void kda_timeline_set_stamps(void* p) { kda::g_stamps = static_cast<unsigned long long*>(p); }\n'
    return src


def build() -> str:
    from linear_attention_decode_kda_amd import build as b

    os.makedirs(OUT, exist_ok=True)
    with open(b.SRC) as f:
        src = _instrument(f.read())
    with open(SRC, "w") as f:
        f.write(src)
    cmd = [b.hipcc(), *b.HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    return LIB


def run(names) -> None:
    import numpy as np
    import torch

    import linear_attention_decode_kda_amd as kda
    from linear_attention_decode_kda_amd import synth

    if not os.path.exists(LIB):
        raise SystemExit(f"{LIB} is not built: python -m linear_attention_decode_kda_amd.timeline build")
    kda.LIB_PATH = LIB  # this process only: the instrumented copy in place of the library
    lib = kda.load()
    lib.kda_timeline_set_stamps.argtypes = [ctypes.c_void_p]
    lib.kda_timeline_set_stamps.restype = None
    dev = torch.device("cuda:0")
    print("| workload | launch | call span (us) | WG end spread (us) | " +
          " | ".join(NAMES[1:]) + " |")
    print("|---" * (4 + len(NAMES) - 1) + "|")
    per_xcd = []
    for spec in names:
        # "workload" or "workload:key=value,..." with params overrides (schedule=2, ...)
        name, _, over = spec.partition(":")
        kw = {k: int(v) for k, v in (x.split("=") for x in over.split(",") if x)}
        w = synth.WORKLOADS[name]
        p = kda.params_for(w, **kw)
        la = kda.select_launch(p)
        nwg = w.N * w.HV * (128 // la["tile_columns"])
        inp = {k: v.to(dev) for k, v in synth.make_inputs(w).items()}
        out = kda.alloc_outputs(w, dev)
        ws = kda.alloc_workspace(p, dev)
        st = torch.zeros(nwg * 16, dtype=torch.int64, device=dev)
        print(f"[timeline] {name}: {nwg} units", file=sys.stderr, flush=True)
        lib.kda_timeline_set_stamps(None)
        for _ in range(200):  # clocks up
            kda.run(p, inp, out, ws)
        torch.cuda.synchronize()
        lib.kda_timeline_set_stamps(st.data_ptr())
        spans, spreads, phases, xcd = [], [], [], {}
        for _ in range(5):
            st.zero_()
            kda.run(p, inp, out, ws)
            torch.cuda.synchronize()
            a = st.view(nwg, 16).cpu().numpy().astype(np.int64)
            a = a[a[:, 0] > 0]
            t0 = a[:, 0].min()
            end = (a[:, 14] - t0) * 0.01
            spans.append(end.max())
            spreads.append(end.max() - end.min() if len(a) <= 2048 else 0.0)
            cols = [1, 2, 3, 4] + sum([[5 + 2 * t, 6 + 2 * t] for t in range(min(w.T, 4))], []) + [13, 14]
            prev, d = 0, {}
            for c in cols:
                d[c] = float(np.median((a[:, c] - a[:, prev]) * 0.01))
                prev = c
            phases.append(d)
            for x in range(8):
                m = a[:, 15] == x
                if m.any():
                    xcd.setdefault(x, []).append((float(end[m].max()), float(np.median((a[m, 14] - a[m, 0]) * 0.01)),
                                                  int(m.sum())))
        lib.kda_timeline_set_stamps(None)
        launch = f"{la['tile_columns']} col, g{la['column_groups']}, cap {la['max_wg_per_cu']}, " \
                 f"{'queue' if la['schedule'] == 2 else 'grid'}, stores {la['store_policy']}"
        cells = []
        for c in range(1, 15):
            vals = [ph[c] for ph in phases if c in ph]
            cells.append(f"{np.median(vals):.2f}" if vals else "-")
        spread = f"{np.median(spreads):.1f}" if max(spreads) > 0 else "-"
        print(f"| {spec} | {launch} | {np.median(spans):.1f} | {spread} | " + " | ".join(cells) + " |")
        per_xcd.append((spec, xcd))
        del inp, out, st
        torch.cuda.empty_cache()
    print("\nPer XCD (median over the five calls): last unit end (us) / median unit duration (us) / units\n")
    print("| workload | " + " | ".join(f"XCD {x}" for x in range(8)) + " |")
    print("|---" * 9 + "|")
    for name, xcd in per_xcd:
        cells = []
        for x in range(8):
            v = xcd.get(x)
            cells.append("-" if not v else
                         f"{np.median([e for e, _, _ in v]):.1f} / {np.median([u for _, u, _ in v]):.2f} / "
                         f"{int(np.median([n for _, _, n in v]))}")
        print(f"| {name} | " + " | ".join(cells) + " |")


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        print(build())
    elif len(sys.argv) > 2 and sys.argv[1] == "run":
        run(sys.argv[2:])
    else:
        raise SystemExit(__doc__)
