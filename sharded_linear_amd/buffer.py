"""The contiguous param/grad buffer of one rank (llm-infra-atlas "05 · grad/param buffer").

Layout comes from the C ABI's sl_layout_build (reverse definition order, 64-element parameter
starts, buckets closed at bucket_size elements and padded to lcm(dp,128)).  Storage is one
zero-filled bf16 param_data and one zero-filled fp32 grad_data of the padded numel (section 5);
each weight is the view param_data[s:e].view(shape) and its main_grad the view
grad_data[s:e].view(shape).  zero_grad_buffer() zeroes grad_data once per iteration with the
library's fill kernel (section 6.6).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import check, lib
from .ops import sl_grad_buffer_zero


@dataclass
class Bucket:
    offset: int
    numel: int
    numel_unpadded: int


@dataclass
class LayoutResult:
    start: list
    end: list
    bucket_id: list
    buckets: list
    numel: int


def sl_default_bucket_size(dp: int) -> int:
    return int(lib().sl_default_bucket_size(dp))


def sl_bucket_divisor(dp: int, high_busbw: bool = False) -> int:
    return int(lib().sl_bucket_divisor(dp, int(high_busbw)))


def sl_layout_build(numels, param_align: int = 64, bucket_size: int | None = None,
                    divisor: int = 128) -> LayoutResult:
    """Host layout of parameters given in definition order (bucket_size None: one bucket)."""
    n = len(numels)
    I64 = ctypes.c_int64 * max(n, 1)
    I32 = ctypes.c_int32 * max(n, 1)
    num, start, end, bid = I64(*numels), I64(), I64(), I32()
    cap = max(n, 1)
    while True:
        off, bn, bu = (ctypes.c_int64 * cap)(), (ctypes.c_int64 * cap)(), (ctypes.c_int64 * cap)()
        nb, total = ctypes.c_int32(0), ctypes.c_int64(0)
        st = lib().sl_layout_build(n, num, param_align, bucket_size or 0, divisor, start, end, bid, cap,
                                   off, bn, bu, ctypes.byref(nb), ctypes.byref(total))
        if st == -6 and nb.value > cap:          # SL_ECAPACITY: retry with the size it asked for
            cap = nb.value
            continue
        check("sl_layout_build", st)
        break
    return LayoutResult(list(start[:n]), list(end[:n]), list(bid[:n]),
                        [Bucket(off[i], bn[i], bu[i]) for i in range(nb.value)], total.value)


class ParamAndGradBuffer:
    """bf16 param_data + fp32 grad_data for weights given as {name: shape} in definition order."""

    def __init__(self, shapes: dict, device, param_align: int = 64, bucket_size: int | None = -1,
                 dp: int = 1, high_busbw: bool = False):
        if bucket_size == -1:
            bucket_size = sl_default_bucket_size(dp)
        self.names = list(shapes)
        self.shapes = {k: tuple(v) for k, v in shapes.items()}
        numels = [int(torch.Size(self.shapes[k]).numel()) for k in self.names]
        self.layout = sl_layout_build(numels, param_align, bucket_size, sl_bucket_divisor(dp, high_busbw))
        self.numel = self.layout.numel
        self.device = torch.device(device)
        self.param_data = torch.zeros(self.numel, dtype=torch.bfloat16, device=self.device)
        self.grad_data = torch.zeros(self.numel, dtype=torch.float32, device=self.device)
        self.index = {k: (self.layout.start[i], self.layout.end[i], self.layout.bucket_id[i])
                      for i, k in enumerate(self.names)}

    def param(self, name: str) -> torch.Tensor:
        s, e, _ = self.index[name]
        return self.param_data[s:e].view(self.shapes[name])

    def main_grad(self, name: str) -> torch.Tensor:
        s, e, _ = self.index[name]
        return self.grad_data[s:e].view(self.shapes[name])

    def attach(self, name: str, p: torch.nn.Parameter) -> torch.nn.Parameter:
        """Remap p.data onto its param_data view (one copy in) and give it a main_grad view."""
        old = p.data
        if old._base is not None:
            raise ValueError(f"{name}: parameter storage must be its own allocation before remapping")
        view = self.param(name)
        view.copy_(old)
        p.data = view
        p.main_grad = self.main_grad(name)
        p.grad_added_to_main_grad = False
        return p

    def zero_grad_buffer(self) -> None:
        sl_grad_buffer_zero(self.grad_data)
