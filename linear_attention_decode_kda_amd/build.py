"""Compile the gfx950 HIP library in-tree: csrc/kda_verify.hip -> libkda_verify.so, and the
plain C caller examples/verify_from_c.c -> examples/verify_from_c (linked to the library)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "kda_verify.hip")
HDR = os.path.join(ROOT, "include", "kda_verify.h")
QHDR = os.path.join(PKG, "csrc", "kda_queue.h")
LIB = os.path.join(PKG, "libkda_verify.so")
ARCH = "gfx950"
EXAMPLE_SRC = os.path.join(PKG, "examples", "verify_from_c.c")
EXAMPLE = os.path.join(PKG, "examples", "verify_from_c")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep the one counter atomic a plain per-lane atomic: the wave-level rewrite reads
    # its result at once, which stalls the wave on every load still in flight
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Always recompiles; writes the library atomically."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_example(verbose: bool = False) -> str:
    """The C caller, with gcc as C11 (the header must compile as C), linked to the library
    found next to the package by a relative run path. Always recompiles."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = EXAMPLE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(rocm, 'include')}", EXAMPLE_SRC, "-o", tmp,
           f"-L{PKG}", "-lkda_verify", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in (SRC, HDR, QHDR))


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_example(verbose=True))
