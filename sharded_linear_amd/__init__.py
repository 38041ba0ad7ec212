"""MI355X-native TP-sharded linear step: fwd, dgrad and fp32 fused wgrad-accumulate on gfx950.

The compute lives in the HIP library libsharded_linear.so (C ABI in include/sharded_linear.h);
this package only marshals torch tensors into it.  Importing the package does not load the
library; the first call does, and raises if it is not built.
"""
from .ops import (sl_grad_buffer_zero, sl_linear_dgrad, sl_linear_dgrad_mxfp8, sl_linear_dgrad_mxfp8w,
                  sl_linear_fwd, sl_linear_fwd_mxfp8, sl_linear_wgrad_accum, sl_linear_wgrad_accum_mxfp8,
                  sl_linear_wgrad_accum_mxfp8x, sl_mxfp8_quantize, sl_mxfp8_wgrad_workspace_bytes,
                  sl_mxfp8_workspace_bytes, sl_wgrad_workspace_bytes, sl_nvfp4_materialize, sl_mxfp8_dequantize,
                  sl_linear_fwd_nvfp4w, sl_linear_dgrad_nvfp4w, sl_set_tuning, tuning,
                  sl_linear_wgrad_accum_noalloc)
from .buffer import ParamAndGradBuffer, sl_bucket_divisor, sl_default_bucket_size, sl_layout_build
from .autograd import LinearWithGradAccumulation, linear_with_grad_accumulation

__all__ = [
    "sl_grad_buffer_zero", "sl_linear_fwd", "sl_linear_dgrad", "sl_linear_wgrad_accum",
    "sl_wgrad_workspace_bytes", "sl_mxfp8_workspace_bytes", "sl_linear_fwd_mxfp8", "sl_linear_dgrad_mxfp8w",
    "sl_linear_wgrad_accum_mxfp8x", "sl_mxfp8_quantize", "sl_linear_dgrad_mxfp8",
    "sl_mxfp8_wgrad_workspace_bytes", "sl_linear_wgrad_accum_mxfp8", "sl_mxfp8_dequantize", "sl_nvfp4_materialize",
    "sl_linear_fwd_nvfp4w", "sl_linear_dgrad_nvfp4w", "sl_set_tuning", "tuning", "sl_linear_wgrad_accum_noalloc", "ParamAndGradBuffer", "sl_layout_build",
    "sl_default_bucket_size", "sl_bucket_divisor", "LinearWithGradAccumulation",
    "linear_with_grad_accumulation",
]
