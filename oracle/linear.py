"""The TP-sharded linear step in float64: forward, dgrad, and wgrad fused into accumulation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation: T tokens (sequence x micro-batch rows flattened, the [s, b, h] activation viewed as
[s*b, h]); ``in``/``out`` are the shard's input and output features.  The weight shard W is
[out, in] (column-parallel: out = out_full/TP; row-parallel: in = in_full/TP), see [ATLAS-TP]
section 1 "Responsibilities of the two modules".

  forward   Y[T,out]  = X[T,in] . W^T            [ATLAS-TP] section 4.1 (matmul of the total
                                                  input with the transposed weight)
  dgrad     dX[T,in]  = dY[T,out] . W            [ATLAS-TP] section 4.2, step 2
  wgrad     G[out,in] += dY^T . X                [ATLAS-TP] section 4.2, step 4: with gradient
                                                  accumulation fusion the weight gradient GEMM
                                                  adds straight into the fp32 main_grad and no
                                                  separate weight gradient exists
  zeroing   G = 0 once per iteration             [ATLAS-BUF] section 6.6 (zero_grad_buffer)

All products are exact definitions, so the oracle computes them with a float64 matmul over the
exact input values (bf16 widened).  The MXFP8 variants dequantise per 32-element block first,
deq(q, s) = E4M3(q) * 2^(s-127), then apply the same formulas; the NVFP4-weight variants decode
deq(c, s, t) = E2M1(c) * E4M3(s) * t per 16-element block, t the fp32 per-tensor scale.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f64, mxfp8_dequant, nvfp4_dequant


def _f64(a):
    """Accept bf16 bit patterns (uint16) or real arrays; return float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def linear_fwd(X, W):
    """Y = X . W^T  ([ATLAS-TP] section 4.1)."""
    X, W = _f64(X), _f64(W)
    assert X.ndim == 2 and W.ndim == 2 and X.shape[1] == W.shape[1]
    return X @ W.T


def linear_dgrad(dY, W):
    """dX = dY . W  ([ATLAS-TP] section 4.2, the dgrad GEMM)."""
    dY, W = _f64(dY), _f64(W)
    assert dY.ndim == 2 and W.ndim == 2 and dY.shape[1] == W.shape[0]
    return dY @ W


def linear_wgrad(X, dY):
    """One micro-batch's weight gradient dY^T . X (never rounded; [GTP] section 3.1 notes the
    wgrad is always computed in high precision)."""
    X, dY = _f64(X), _f64(dY)
    assert X.shape[0] == dY.shape[0]
    return dY.T @ X


def linear_wgrad_accum(main_grad, X, dY):
    """main_grad + dY^T . X, the fused accumulate ([ATLAS-TP] section 4.2, step 4)."""
    return np.asarray(main_grad, dtype=np.float64) + linear_wgrad(X, dY)


def step(W, Xs, dYs, main_grad0=None):
    """One iteration over micro-batches k = 1..m with a fixed weight shard.

    main_grad starts at zero (zero_grad_buffer, [ATLAS-BUF] section 6.6) unless given, and every
    micro-batch adds into it with no reduction in between (no_sync, [ATLAS-BUF] section 6.4).
    Returns (list of Y_k, list of dX_k, final main_grad).
    """
    W = _f64(W)
    G = np.zeros(W.shape) if main_grad0 is None else np.asarray(main_grad0, dtype=np.float64).copy()
    Ys, dXs = [], []
    for X, dY in zip(Xs, dYs):
        Ys.append(linear_fwd(X, W))
        dXs.append(linear_dgrad(dY, W))
        G = linear_wgrad_accum(G, X, dY)
    return Ys, dXs, G


# ---- brute force: pure-Python triple loops, for tiny shapes only --------------------------------

def fwd_brute(X, W):
    X, W = _f64(X), _f64(W)
    T, n_in = X.shape
    n_out = W.shape[0]
    Y = np.zeros((T, n_out))
    for t in range(T):
        for o in range(n_out):
            s = 0.0
            for i in range(n_in):
                s += float(X[t, i]) * float(W[o, i])
            Y[t, o] = s
    return Y


def dgrad_brute(dY, W):
    dY, W = _f64(dY), _f64(W)
    T, n_out = dY.shape
    n_in = W.shape[1]
    dX = np.zeros((T, n_in))
    for t in range(T):
        for i in range(n_in):
            s = 0.0
            for o in range(n_out):
                s += float(dY[t, o]) * float(W[o, i])
            dX[t, i] = s
    return dX


def wgrad_accum_brute(main_grad, X, dY):
    X, dY = _f64(X), _f64(dY)
    G = np.array(main_grad, dtype=np.float64, copy=True)
    T = X.shape[0]
    for o in range(G.shape[0]):
        for i in range(G.shape[1]):
            s = 0.0
            for t in range(T):
                s += float(dY[t, o]) * float(X[t, i])
            G[o, i] += s
    return G


# ---- MXFP8 operand variants ([GTP] section 1.3: E4M3 data with one E8M0 scale per 32 elements) --

def linear_fwd_mxfp8(Xq, Xs, Wq, Ws):
    """Y = deq(Xq, Xs) . deq(Wq, Ws)^T; both blocks run along ``in`` (the contraction axis)."""
    return linear_fwd(mxfp8_dequant(Xq, Xs), mxfp8_dequant(Wq, Ws))


def linear_dgrad_mxfp8w(dY, Wq, Ws):
    """dX = dY . deq(Wq, Ws), dY in bf16."""
    return linear_dgrad(dY, mxfp8_dequant(Wq, Ws))


def linear_wgrad_accum_mxfp8x(main_grad, Xq, Xs, dY):
    """main_grad + dY^T . deq(Xq, Xs), dY in bf16."""
    return linear_wgrad_accum(main_grad, mxfp8_dequant(Xq, Xs), dY)


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| over one tensor: the parity metric of this step."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# ---- MXFP8 backward as well ([GTP] section 1.3: forward and backward GEMMs in MXFP8, each GEMM
# reading copies quantised along its own contraction axis; the weight gradient is accumulated in
# fp32 as above) --------------------------------------------------------------------------------

def linear_dgrad_mxfp8(dYq, dYs, WqT, WsT):
    """dX = deq(dY rowwise) . deq(W columnwise): dY quantised along ``out`` ([T, out] codes), W
    quantised along ``out`` and stored transposed ([in, out] codes)."""
    return mxfp8_dequant(dYq, dYs) @ mxfp8_dequant(WqT, WsT).T


def linear_wgrad_accum_mxfp8(main_grad, dYqT, dYsT, XqT, XsT):
    """main_grad + deq(dY columnwise) . deq(X columnwise)^T: both quantised along T and stored
    transposed ([out, T] and [in, T] codes)."""
    return np.asarray(main_grad, dtype=np.float64) + mxfp8_dequant(dYqT, dYsT) @ mxfp8_dequant(XqT, XsT).T


# ---- NVFP4 weights ([GTP] section 1.3, "Native NVFP4 param": the weight shard lives as packed
# E2M1 with block-16 scales and a per-tensor scale; activations and gradients stay bf16) ---------

def linear_fwd_nvfp4w(X, Wq, Ws, w_scale):
    """Y = X . deq(W)^T with W in NVFP4."""
    return linear_fwd(X, nvfp4_dequant(Wq, Ws, w_scale))


def linear_dgrad_nvfp4w(dY, Wq, Ws, w_scale):
    """dX = dY . deq(W) with W in NVFP4."""
    return linear_dgrad(dY, nvfp4_dequant(Wq, Ws, w_scale))
