"""Build libw4_bench.so, the measurement-only kernels bench.py uses (a plain copy
of known size for calibrating rocprofv3's byte counters, and a streaming read
that gives the practical read bandwidth), in this folder with hipcc for gfx950.

It is not part of the product library (bit_group_quantized_w4_amd/libw4.so)
and nothing in the product loads it.

Usage: python bench_support/build.py   (or __graft_entry__.build()).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libw4_bench.so")
SOURCES = ["copy_probe.hip"]
ARCH = "gfx950"


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4_bench.so)")


def build(verbose=True):
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip"] + [os.path.join(HERE, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def built():
    return os.path.exists(LIB)


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
