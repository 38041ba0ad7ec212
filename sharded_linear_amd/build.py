"""Build the HIP C-ABI library in-tree for gfx950.

    python -m sharded_linear_amd.build        # -> sharded_linear_amd/libsharded_linear.so

hipcc compiles the kernels (cross-compiles without a GPU) and the host layout builder, one object
per source (the bf16 GEMM source in three parts) in parallel, and links them into one shared
library.  Every HIP source gets -packed-fp32-ops disabled: the library relies on scalar and float2
arithmetic only.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile
import time

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


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose:
        print(f"[{time.time() - t0:5.1f}s] " + " ".join(cmd), flush=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then link."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="sl_build_") as tmpdir:
        objs, jobs = [], []
        for src in SOURCES:
            # the bf16 GEMM instantiations compile as three parts (fwd, dgrad, wgrad) in parallel
            parts = [[f"-DSL2_PART={k}"] for k in (1, 2, 3)] if src.endswith("sl_gemm2.hip") else [[]]
            for i, extra in enumerate(parts):
                obj = os.path.join(tmpdir, f"{os.path.basename(src)}.{i}.o")
                objs.append(obj)
                jobs.append([cc, *_flags(), *extra, "-c", src, "-o", obj])
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
