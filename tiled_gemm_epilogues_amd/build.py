"""Builds the HIP library tiled_gemm_epilogues_amd/libtge.so for gfx950 with hipcc.

The kernel source is compiled once per (input, output) type pair, in parallel, and linked with
the host API into one shared library that exports the C ABI declared in include/gemm.h.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtge.so")

PAIRS = ["F32_F32", "F16_F16", "F16_F32", "BF16_BF16", "BF16_F32", "I8_I32"]
FAST_PAIRS = ["F16_F16", "F16_F32", "BF16_BF16", "BF16_F32", "I8_I32"]
SKINNY_PAIRS = ["F16_F16", "F16_F32", "BF16_BF16", "BF16_F32", "I8_I32"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # never let the compiler form packed fp32 VALU instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    steps = []
    for pair in PAIRS:
        obj = os.path.join(BUILD, f"gemm_kernels_{pair.lower()}.o")
        steps.append([HIPCC, *FLAGS, f"-DTGE_PAIR_{pair}", "-c",
                      os.path.join(CSRC, "gemm_kernels.hip"), "-o", obj])
    for pair in FAST_PAIRS:
        obj = os.path.join(BUILD, f"gemm_fast_{pair.lower()}.o")
        steps.append([HIPCC, *FLAGS, f"-DTGE_PAIR_{pair}", "-c",
                      os.path.join(CSRC, "gemm_fast.hip"), "-o", obj])
    for pair in SKINNY_PAIRS:
        obj = os.path.join(BUILD, f"gemm_skinny_{pair.lower()}.o")
        steps.append([HIPCC, *FLAGS, f"-DTGE_PAIR_{pair}", "-c",
                      os.path.join(CSRC, "gemm_skinny.hip"), "-o", obj])
    for name in ("gemm_complex", "gemm_diag", "gemm_repack"):
        steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, name + ".hip"), "-o",
                      os.path.join(BUILD, name + ".o")])
    api_obj = os.path.join(BUILD, "gemm_api.o")
    steps.append([HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "gemm_api.cpp"), "-o", api_obj])
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    objs = [s[-1] for s in steps]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
