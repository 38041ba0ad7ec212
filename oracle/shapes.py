"""Parameter counts of the Llama-3.2-1B-shape ledger and the TP=2 shard shapes of the step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[MEGA-SRC] section 1 ("Overview"): L=16 layers, h=2048, f=8192, n_q=32, n_kv=8, d_h=64,
v=128256, untied embedding and output layer; per layer the Q,K,V,O weights hold
2h^2 + 2h(n_kv d_h) parameters, SwiGLU gate/up/down hold 3hf, plus two RMSNorm weights (2h).
"""
from __future__ import annotations

LLAMA_1B = dict(L=16, h=2048, f=8192, n_q=32, n_kv=8, d_h=64, v=128256)


def per_layer_params(h, f, n_kv, d_h, **_):
    """2h^2 + 2h*n_kv*d_h + 3hf + 2h."""
    return 2 * h * h + 2 * h * n_kv * d_h + 3 * h * f + 2 * h


def total_params(L, h, f, n_kv, d_h, v, **_):
    """L * per-layer + untied input embedding and output layer (v*h each) + final RMSNorm (h).

    The page lists 16 layers, two v*h matrices and a total about 1,498,482,688; that total is
    exactly h larger than the first two terms, which is the final norm weight of the model.
    """
    return L * per_layer_params(h, f, n_kv, d_h) + 2 * v * h + h


def tp_shard_shapes(h, f, n_q, n_kv, d_h, tp=2, **_):
    """Weight shards [out, in] of one layer on one TP rank, in definition order.

    Column-parallel (split along out): fused QKV [(n_q + 2 n_kv) d_h / tp, h] and fused
    gate/up [2f/tp, h].  Row-parallel (split along in): O [h, n_q d_h / tp], down [h, f/tp].
    ([ATLAS-TP] section 1: column weight is [out/TP, in], row weight is [out, in/TP].)
    """
    return {
        "linear_qkv": ((n_q + 2 * n_kv) * d_h // tp, h),
        "linear_proj": (h, n_q * d_h // tp),
        "linear_fc1": (2 * f // tp, h),
        "linear_fc2": (h, f // tp),
    }
