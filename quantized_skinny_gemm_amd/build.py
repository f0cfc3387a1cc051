"""Builds libqsgemm.so (gfx950 only) in-tree with hipcc.

    python quantized_skinny_gemm_amd/build.py      (or __graft_entry__.build())

It is run by path, not as ``-m quantized_skinny_gemm_amd.build``: importing
the package loads the library this script is about to replace.

Each HIP source is compiled to an object under ``_build/`` in parallel and
the objects are linked into ``quantized_skinny_gemm_amd/libqsgemm.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqsgemm.so")
# bench.py's read-ceiling probe: a separate library, not part of the C ABI
BENCH_SRC = os.path.join(ROOT, "bench_read.hip")
BENCH_LIB = os.path.join(ROOT, "bench_read.so")

HIP_SOURCES = ["api.hip", "quantize.hip", "q4_narrow.hip", "q4_mma.hip", "q4_skinny.hip",
               "q4_wide_i8.hip", "f_kernels.hip", "repack.hip"]
CXX_SOURCES = ["plan.cpp", "dispatch_table.cpp"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU ops stay disabled (no v_pk_*_f32 in any kernel)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the scale epilogues read every output
    # register, and an accumulation-register result costs one extra move each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the leading kernel arguments (up to 14 dwords) arrive in scalar
    # registers at wave launch instead of through a load from the kernel
    # argument segment: a wave can address its first loads at once
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
    "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout + r.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-ldl", "-o", tmp])
    os.replace(tmp, LIB)
    if os.path.exists(BENCH_SRC):
        tmp = BENCH_LIB + ".tmp"
        _run([hipcc, *HIPCC_FLAGS, "-shared", BENCH_SRC, "-o", tmp])
        os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
