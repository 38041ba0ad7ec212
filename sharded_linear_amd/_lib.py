"""ctypes loader of libsharded_linear.so with the prototypes of include/sharded_linear.h.

The library must share torch's HIP runtime (streams and device pointers cross the boundary), so
torch is imported first; the loader then checks that exactly one libamdhip64 is mapped.  There
is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime before ours resolves against it)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsharded_linear.so")

c_i32, c_i64, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
P_I64 = ctypes.POINTER(ctypes.c_int64)
P_I32 = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/sharded_linear.h
PROTOTYPES = {
    "sl_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sl_set_tuning": (ctypes.c_int, [c_i32, c_i32, P_I32]),
    "sl_layout_build": (ctypes.c_int, [c_i32, P_I64, c_i64, c_i64, c_i64, P_I64, P_I64, P_I32, c_i32,
                                       P_I64, P_I64, P_I64, P_I32, P_I64]),
    "sl_default_bucket_size": (c_i64, [c_i64]),
    "sl_bucket_divisor": (c_i64, [c_i64, c_i32]),
    "sl_grad_buffer_zero": (ctypes.c_int, [c_vp, c_vp, c_i64]),
    "sl_linear_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64]),
    "sl_linear_dgrad": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64]),
    "sl_wgrad_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "sl_linear_wgrad_accum": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_sz]),
    "sl_linear_wgrad_accum_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64]),
    "sl_linear_fwd_mxfp8": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64]),
    "sl_mxfp8_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "sl_linear_dgrad_mxfp8w": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_sz]),
    "sl_linear_wgrad_accum_mxfp8x": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                                    c_vp, c_sz]),
    "sl_mxfp8_quantize": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "sl_linear_dgrad_mxfp8": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64]),
    "sl_mxfp8_wgrad_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "sl_linear_wgrad_accum_mxfp8": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                                   c_vp, c_sz]),
    "sl_mxfp8_dequantize": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64]),
    "sl_nvfp4_materialize": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64]),
    "sl_linear_fwd_nvfp4w": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_i64, c_i64, c_i64]),
    "sl_linear_dgrad_nvfp4w": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_i64, c_i64, c_i64]),
}

_lib = None


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process."""
    with open("/proc/self/maps") as f:
        return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sharded_linear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        rt = hip_runtimes_mapped()
        if len(rt) > 1:
            raise RuntimeError(f"two HIP runtimes mapped ({rt}); streams and pointers would not be shared")
        _lib = L
    return _lib


class SLError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().sl_status_str(status).decode()}")


def check(fn: str, status: int) -> None:
    if status != 0:
        raise SLError(fn, status)
