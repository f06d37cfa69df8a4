"""Build libsqg.so in-tree for gfx950 with hipcc (no JIT, no torch extension).

Usage: python -m streamed_qkv_gemm_amd.build   (or call build()).
Objects go to streamed_qkv_gemm_amd/_build/, the library to
streamed_qkv_gemm_amd/libsqg.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsqg.so")

ARCH = "gfx950"
HIP_SOURCES = ["qkv_quant.hip", "packed_attention.hip", "test_kernels.hip", "runtime.hip"]
HOST_SOURCES = ["sqg_api.cpp"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I" + CSRC, "-I" + os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
              "-I" + CSRC, "-I" + os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsqg.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed (%d):\n%s\n%s" % (r.returncode, " ".join(cmd), r.stdout))
    if verbose and r.stdout.strip():
        print(r.stdout, flush=True)
    return r.stdout


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link libsqg.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    cxx = shutil.which("g++") or "g++"
    steps = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        steps.append([hipcc] + HIP_FLAGS + ["-c", os.path.join(CSRC, s), "-o", obj])
    for s in HOST_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        steps.append([cxx] + HOST_FLAGS + ["-c", os.path.join(CSRC, s), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
