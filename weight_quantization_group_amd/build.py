"""Build the HIP library ``libhqq.so`` for gfx950, in-tree.

    python -m weight_quantization_group_amd.build

The translation units are compiled in parallel (one hipcc process each) and
linked into one shared library.  Flags that matter for exactness:
  -ffp-contract=off                  no fma contraction beyond the explicit ones
  -fno-gpu-flush-denormals-to-zero   fp32 denormals kept (IEEE)
  (HIP's default fp32 division is correctly rounded; no unsafe-math flags)
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed-fp32 VALU ops
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhqq.so")

SOURCES = ["hqq_abi.cpp", "hqq_stream.cpp", "hqq_solve.hip", "hqq_solve_b1.hip", "hqq_solve_b2.hip",
           "hqq_solve_b3.hip", "hqq_solve_b4.hip", "hqq_solve_b8.hip",
           "hqq_solve_b1_bf16.hip", "hqq_solve_b2_bf16.hip", "hqq_solve_b3_bf16.hip",
           "hqq_solve_b4_bf16.hip", "hqq_solve_b8_bf16.hip", "hqq_codec.hip",
           "hqq_linear.hip", "hqq_gemm.cpp"]

FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-pass-failed",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lhipblaslt"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
