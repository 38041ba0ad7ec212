"""Workloads of the TP-sharded linear step: shard shapes, tokens and micro-batches, and their
seeded synthetic inputs.

Shapes follow the Llama-3.2-1B-shape ledger of arganzheng.life "Megatron-LM architecture and
source guide" section 1 (h=2048, f=8192, 32 q heads, 8 kv heads, d_h=64; seq 8192, micro-batch 1)
at TP=2, and a 7B-class layer (h=4096, ffn=11008) at TP=2 with 4096 tokens x micro-batch 2.
Weights are [out, in] shards, listed in model definition order (the buffer lays them out
reversed).  Inputs of every GEMM are independent draws (the activation between the linears is
not part of the step).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import ROLE_DY, ROLE_W, ROLE_X, W_STD, mxfp8_normal, normal_bf16, nvfp4_normal, seed_for


@dataclass(frozen=True)
class Workload:
    key: str
    index: int                     # config number used in the seeds
    title: str
    params: dict                   # name -> (out, in), definition order
    tokens: int                    # T rows per micro-batch
    microbatches: int
    timed: tuple = ()              # params whose GEMMs form the step (default: all)
    mxfp8: bool = False            # W and X quantised to MXFP8, dY bf16
    mxfp8_all: bool = False        # bf16 inputs, quantised to MXFP8 inside the step (all GEMMs fp8)
    nvfp4w: bool = False           # W stored as NVFP4 (packed E2M1, E4M3 per 16, fp32 tensor scale)
    extra: dict = field(default_factory=dict)

    @property
    def step_params(self):
        return self.timed or tuple(self.params)

    def flops_per_step(self) -> int:
        """Algorithmic FLOPs: 2*T*in*out per GEMM, three GEMMs per param per micro-batch."""
        return sum(6 * self.tokens * o * i for o, i in (self.params[p] for p in self.step_params)) * self.microbatches


LLAMA1B_TP2 = {"linear_qkv": (1536, 2048), "linear_proj": (2048, 1024),
               "linear_fc1": (8192, 2048), "linear_fc2": (2048, 4096)}
LAYER7B_TP2 = {"linear_qkv": (6144, 4096), "linear_proj": (4096, 2048),
               "linear_fc1": (11008, 4096), "linear_fc2": (4096, 5504)}

WORKLOADS = {
    "c1": Workload("c1", 1, "tiny TP=1 linear, 128 tokens, 2 micro-batches",
                   {"weight": (512, 256)}, 128, 2),
    "c2": Workload("c2", 2, "Llama-3.2-1B-shape MLP TP=2 shard, seq 8192 x mb 1, 8 micro-batches",
                   {"linear_fc1": LLAMA1B_TP2["linear_fc1"], "linear_fc2": LLAMA1B_TP2["linear_fc2"]}, 8192, 8),
    "c3": Workload("c3", 3, "Llama-3.2-1B-shape attention projections TP=2 shard, 8192 tokens",
                   dict(LLAMA1B_TP2), 8192, 1, timed=("linear_qkv", "linear_proj")),
    "c4": Workload("c4", 4, "7B-class dense layer TP=2 shard, 4096 tokens x mb 2",
                   dict(LAYER7B_TP2), 8192, 1),
    "c5": Workload("c5", 5, "Llama-3.2-1B-shape MLP TP=2 shard with MXFP8 W and X, 8 micro-batches",
                   {"linear_fc1": LLAMA1B_TP2["linear_fc1"], "linear_fc2": LLAMA1B_TP2["linear_fc2"]}, 8192, 8,
                   mxfp8=True),
    # the next step of the low-precision path: every GEMM in MXFP8, dY quantised as well
    "c6": Workload("c6", 6, "Llama-3.2-1B-shape MLP TP=2 shard, all GEMMs MXFP8 (X, W, dY quantised in the step), "
                   "8 micro-batches",
                   {"linear_fc1": LLAMA1B_TP2["linear_fc1"], "linear_fc2": LLAMA1B_TP2["linear_fc2"]}, 8192, 8,
                   mxfp8_all=True),
    # native NVFP4 weights: the shard stays NVFP4, activations and gradients bf16
    "c7": Workload("c7", 7, "Llama-3.2-1B-shape MLP TP=2 shard with NVFP4 weights, 8 micro-batches",
                   {"linear_fc1": LLAMA1B_TP2["linear_fc1"], "linear_fc2": LLAMA1B_TP2["linear_fc2"]}, 8192, 8,
                   nvfp4w=True),
}


def _pidx(w: Workload, name: str) -> int:
    return list(w.params).index(name)


def weight(w: Workload, name: str):
    """bf16 bits [out, in]; (codes, scales) for MXFP8 workloads; (packed codes, scales, tensor
    scale) for NVFP4-weight workloads."""
    shape = w.params[name]
    seed = seed_for(w.index, _pidx(w, name), 0, ROLE_W)
    if w.nvfp4w:
        return nvfp4_normal(shape, seed, W_STD)
    return mxfp8_normal(shape, seed, W_STD) if w.mxfp8 else normal_bf16(shape, seed, W_STD)


def x(w: Workload, name: str, mb: int):
    """Input [T, in] of micro-batch mb: bf16 bits, or (codes, scales) for MXFP8 workloads."""
    shape = (w.tokens, w.params[name][1])
    seed = seed_for(w.index, _pidx(w, name), mb, ROLE_X)
    return mxfp8_normal(shape, seed) if w.mxfp8 else normal_bf16(shape, seed)


def dy(w: Workload, name: str, mb: int):
    """Output gradient [T, out] of micro-batch mb, bf16 bits."""
    shape = (w.tokens, w.params[name][0])
    return normal_bf16(shape, seed_for(w.index, _pidx(w, name), mb, ROLE_DY))
