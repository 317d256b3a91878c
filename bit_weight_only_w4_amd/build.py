"""Build the W4 HIP library (libw4.so) in-tree for gfx950.

Usage: python -m bit_weight_only_w4_amd.build   (or call build()).
Every HIP translation unit is compiled with hipcc for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libw4.so")
SOURCES = ["w4_api.cpp", "w4_gemv.hip",
           "w4_gemv_nf4_f16.hip", "w4_gemv_nf4_bf16.hip", "w4_gemv_int4_f16.hip",
           "w4_gemv_int4_bf16.hip", "w4_gemv_fp4_f16.hip", "w4_gemv_fp4_bf16.hip",
           "w4_gemv_nf4_f16_grouped.hip", "w4_gemv_nf4_bf16_grouped.hip",
           "w4_gemv_int4_f16_grouped.hip", "w4_gemv_int4_bf16_grouped.hip",
           "w4_gemv_fp4_f16_grouped.hip", "w4_gemv_fp4_bf16_grouped.hip",
           "w4_gemv_int4a_f16.hip", "w4_gemv_int4a_bf16.hip", "w4_gemv_int4a_f16_grouped.hip",
           "w4_gemv_int4a_bf16_grouped.hip",
           "w4_quant.hip", "w4_twopass.hip", "w4_mfma.hip", "w4_mfma_grouped.hip", "w4_gemm.hip", "w4_gemm_fold.hip",
           "w4_gptq.hip", "w4_sparse24.hip", "w4_probe.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the W4 library)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
