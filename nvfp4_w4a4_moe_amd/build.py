"""In-tree build of libnv4moe.so for gfx950 with hipcc.

    python -m nvfp4_w4a4_moe_amd.build            # build (always recompiles)

Every HIP translation unit is compiled with the flags the numerics rely on:
correctly rounded FP32 division, FP32 denormals kept, no floating-point
contraction, and packed FP32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnv4moe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("NV4_OFFLOAD_ARCH", "gfx950")

# the grouped GEMM's instantiations come first: they take the longest to compile
SOURCES = ["gemm_m_swiglu.hip", "gemm_m.hip", "gemm_k.hip", "gemm_m_ksplit.hip", "gemm_m_swiglu_rows.hip", "gemm_m_rows.hip",
           "gemm_m_small.hip", "gemm_m_wf16.hip", "gemm_m_wf16_ksplit.hip",
           "gemm_bf16.hip", "gemm.hip", "quantize.hip", "permute.hip", "convert.hip", "combine.hip", "ceilings.hip", "api.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(max(os.cpu_count() or 1, 1), 16, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
