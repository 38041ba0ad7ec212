"""Autograd function of the linear step with gradient-accumulation fusion.

llm-infra-atlas "01 · ColumnParallelLinear / RowParallelLinear and the core autograd",
section 4: forward saves (input, weight) and computes Y = X.W^T; backward computes the input
gradient dY.W, then the weight gradient straight into the fp32 weight.main_grad, returns no
weight gradient and marks weight.grad_added_to_main_grad.  Communication (sequence-parallel
all-gather, dgrad all-reduce / reduce-scatter) is outside this single-GPU step.
"""
from __future__ import annotations

import torch

from .ops import sl_linear_dgrad, sl_linear_fwd, sl_linear_wgrad_accum


class LinearWithGradAccumulation(torch.autograd.Function):
    @staticmethod
    def forward(ctx, input: torch.Tensor, weight: torch.Tensor):
        if not hasattr(weight, "main_grad"):
            raise ValueError("gradient accumulation fusion needs weight.main_grad (a grad_data view)")
        x2 = input.reshape(-1, input.shape[-1])
        y = sl_linear_fwd(x2.contiguous(), weight.detach())
        ctx.save_for_backward(input, weight)
        return y.view(*input.shape[:-1], weight.shape[0])

    @staticmethod
    def backward(ctx, grad_output: torch.Tensor):
        input, weight = ctx.saved_tensors
        dy = grad_output.reshape(-1, grad_output.shape[-1]).contiguous()
        x2 = input.reshape(-1, input.shape[-1]).contiguous()
        dx = sl_linear_dgrad(dy, weight.detach())
        sl_linear_wgrad_accum(x2, dy, weight.main_grad)
        weight.grad_added_to_main_grad = True
        return dx.view(*input.shape), None


def linear_with_grad_accumulation(input: torch.Tensor, weight: torch.Tensor) -> torch.Tensor:
    return LinearWithGradAccumulation.apply(input, weight)
