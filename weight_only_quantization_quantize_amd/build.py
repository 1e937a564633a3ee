"""Build libwoq.so (every HIP kernel plus the C ABI) for gfx950 with hipcc.

Run as ``python -m weight_only_quantization_quantize_amd.build``; the library is
written next to this file so it travels with the source tree.  Each call
recompiles every translation unit.
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
LIB = os.path.join(HERE, "libwoq.so")
ARCH = os.environ.get("WOQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["woq_api.cpp", "quantize_pack.hip", "gemv.hip", "gemm.hip", "gemm_lds.hip", "gemm_regb.hip", "gemm_mid.hip", "gemm_mid_bf16.hip", "gemm_skinny.hip", "dequantize.hip",
           "awq_search.hip", "gptq.hip", "probes.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed-FP32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division: the quantizer's code decisions rely on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libwoq")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
