"""Build libw4.so in-tree with hipcc for gfx950.

Usage: python bit_group_quantized_w4_amd/_build.py   (or __graft_entry__.build()).
Run it as a script (not with -m): importing the package loads the library,
which may be missing or stale before this builds it.
The shared objects land next to this file, so a snapshot of the repository
carries them to a GPU host without any JIT cache.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB = os.path.join(PKG, "libw4.so")

LIB_SOURCES = ["abi.cpp", "quantize.hip", "linear.hip", "awq.hip", "gptq.hip", "dense.hip"]

ARCH = "gfx950"


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Wno-unused-function",
        # keep fp32 math IEEE: no fast-math, no denormal flushing, no
        # reciprocal division; packed fp32 instructions stay off.
        "-fno-fast-math",
        "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: the per-group scaling reads them with
        # plain VALU instead of v_accvgpr_read copies.
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # the first 16 dwords of scalar kernel arguments arrive preloaded in
        # SGPRs, so single-linear and quantize kernels start issuing loads
        # without a kernel-argument fetch.
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _compile(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc()] + common_flags() + ["-x", "hip"] + [os.path.join(CSRC, s) for s in sources] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose=True):
    _compile(LIB_SOURCES, LIB, verbose)
    return LIB


def built():
    return os.path.exists(LIB)


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
