"""Build the HIP C-ABI library in-tree for gfx950.

    python -m sharded_linear_amd.build        # -> sharded_linear_amd/libsharded_linear.so

hipcc compiles the kernels (cross-compiles without a GPU) and the host layout builder into one
shared library.  Every HIP source gets -packed-fp32-ops disabled: the library relies on scalar
and float2 arithmetic only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsharded_linear.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("sl_gemm.hip", "sl_gemm2.hip", "sl_gemm_f8.hip", "sl_quant.hip", "sl_nvfp4.hip", "sl_layout.cpp")]
ARCH = os.environ.get("SL_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
