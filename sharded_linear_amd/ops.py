"""Thin torch binding of the C ABI: argument marshalling only, every step runs in the HIP library.

Function names match the C entry points.  Tensors must be CUDA (HIP) tensors on one device,
contiguous, with the dtypes of include/sharded_linear.h; work is enqueued on torch's current
stream of that device.  Outputs not supplied are allocated with torch.empty (plumbing).
"""
from __future__ import annotations

import contextlib
import ctypes

import torch

from ._lib import check, lib

BF16, F32, U8 = torch.bfloat16, torch.float32, torch.uint8


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _want(t, name, dtype, shape, dev):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device(t):
    if not t.is_cuda:
        raise ValueError("the HIP library works on GPU tensors only; got a CPU tensor")
    return t.device


# knobs of sl_set_tuning, in the order of the header's SL_TUNE_* enum
TUNE_KNOBS = {"fwd": 0, "dgrad": 1, "wgrad": 2, "splitk": 3, "f8": 4}


def sl_set_tuning(knob: str, value: int) -> int:
    """Force a tuning choice (-1 restores the built-in one); returns the previous value."""
    prev = ctypes.c_int32(0)
    check("sl_set_tuning", lib().sl_set_tuning(TUNE_KNOBS[knob], int(value), ctypes.byref(prev)))
    return prev.value


@contextlib.contextmanager
def tuning(**knobs):
    """Within the block, force the given knobs (names of TUNE_KNOBS; ``gemm=n`` sets the tile
    configuration of all three bf16 products, so it takes 0..24; the forward-only 256x192
    configuration 25 is forced with ``fwd=25``); the previous values come back on exit."""
    if "gemm" in knobs:
        cfg = knobs.pop("gemm")
        knobs = {"fwd": cfg, "dgrad": cfg, "wgrad": cfg, **knobs}
    saved = []
    try:
        for k, v in knobs.items():
            saved.append((k, sl_set_tuning(k, v)))
        yield
    finally:
        for k, v in reversed(saved):
            sl_set_tuning(k, v)


def sl_grad_buffer_zero(grad_data: torch.Tensor) -> torch.Tensor:
    dev = _device(grad_data)
    _want(grad_data, "grad_data", F32, (grad_data.numel(),), dev)
    check("sl_grad_buffer_zero", lib().sl_grad_buffer_zero(_stream(dev), _ptr(grad_data), grad_data.numel()))
    return grad_data


def sl_linear_fwd(X: torch.Tensor, W: torch.Tensor, Y: torch.Tensor | None = None) -> torch.Tensor:
    """Y[T,out] = X[T,in] . W[out,in]^T (bf16)."""
    dev = _device(X)
    T, n_in = X.shape
    n_out = W.shape[0]
    _want(X, "X", BF16, (T, n_in), dev)
    _want(W, "W", BF16, (n_out, n_in), dev)
    if Y is None:
        Y = torch.empty((T, n_out), dtype=BF16, device=dev)
    _want(Y, "Y", BF16, (T, n_out), dev)
    check("sl_linear_fwd", lib().sl_linear_fwd(_stream(dev), _ptr(X), _ptr(W), _ptr(Y), T, n_in, n_out))
    return Y


def sl_linear_dgrad(dY: torch.Tensor, W: torch.Tensor, dX: torch.Tensor | None = None) -> torch.Tensor:
    """dX[T,in] = dY[T,out] . W[out,in] (bf16)."""
    dev = _device(dY)
    T, n_out = dY.shape
    n_in = W.shape[1]
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(W, "W", BF16, (n_out, n_in), dev)
    if dX is None:
        dX = torch.empty((T, n_in), dtype=BF16, device=dev)
    _want(dX, "dX", BF16, (T, n_in), dev)
    check("sl_linear_dgrad", lib().sl_linear_dgrad(_stream(dev), _ptr(dY), _ptr(W), _ptr(dX), T, n_in, n_out))
    return dX


def sl_wgrad_workspace_bytes(T: int, n_in: int, n_out: int) -> int:
    return int(lib().sl_wgrad_workspace_bytes(T, n_in, n_out))


_WS = {}


def wgrad_workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    """A workspace of at least ``nbytes`` for the current stream of ``dev`` (contents never
    matter to the kernels); one buffer per stream is reused and only grows."""
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=U8, device=dev)
        _WS[key] = ws
    return ws


def sl_linear_wgrad_accum(X: torch.Tensor, dY: torch.Tensor, main_grad: torch.Tensor,
                          workspace: torch.Tensor | None = None) -> torch.Tensor:
    """main_grad[out,in] += dY[T,out]^T . X[T,in] in fp32, in place."""
    dev = _device(X)
    T, n_in = X.shape
    n_out = dY.shape[1]
    _want(X, "X", BF16, (T, n_in), dev)
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(main_grad, "main_grad", F32, (n_out, n_in), dev)
    need = sl_wgrad_workspace_bytes(T, n_in, n_out)
    if workspace is None:
        workspace = wgrad_workspace(dev, need) if need else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("sl_linear_wgrad_accum", lib().sl_linear_wgrad_accum(
        _stream(dev), _ptr(X), _ptr(dY), _ptr(main_grad), T, n_in, n_out, _ptr(workspace), nbytes))
    return main_grad


def sl_linear_wgrad_accum_noalloc(X: torch.Tensor, dY: torch.Tensor, main_grad: torch.Tensor) -> torch.Tensor:
    """main_grad += dY^T . X in fp32, in place, with the split-K planes in the library's own device
    array (no workspace, no allocation)."""
    dev = _device(X)
    T, n_in = X.shape
    n_out = dY.shape[1]
    _want(X, "X", BF16, (T, n_in), dev)
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(main_grad, "main_grad", F32, (n_out, n_in), dev)
    check("sl_linear_wgrad_accum_noalloc", lib().sl_linear_wgrad_accum_noalloc(
        _stream(dev), _ptr(X), _ptr(dY), _ptr(main_grad), T, n_in, n_out))
    return main_grad


def sl_linear_fwd_mxfp8(Xq, Xs, Wq, Ws, Y=None):
    """Y = deq(Xq, Xs) . deq(Wq, Ws)^T (bf16 out); codes and scales are uint8."""
    dev = _device(Xq)
    T, n_in = Xq.shape
    n_out = Wq.shape[0]
    _want(Xq, "Xq", U8, (T, n_in), dev)
    _want(Xs, "Xs", U8, (T, n_in // 32), dev)
    _want(Wq, "Wq", U8, (n_out, n_in), dev)
    _want(Ws, "Ws", U8, (n_out, n_in // 32), dev)
    if Y is None:
        Y = torch.empty((T, n_out), dtype=BF16, device=dev)
    _want(Y, "Y", BF16, (T, n_out), dev)
    check("sl_linear_fwd_mxfp8", lib().sl_linear_fwd_mxfp8(
        _stream(dev), _ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), _ptr(Y), T, n_in, n_out))
    return Y


def sl_mxfp8_workspace_bytes(T: int, n_in: int, n_out: int) -> int:
    return int(lib().sl_mxfp8_workspace_bytes(T, n_in, n_out))


def sl_linear_dgrad_mxfp8w(dY, Wq, Ws, dX=None, workspace=None):
    """dX = dY . deq(Wq, Ws) (bf16 in/out)."""
    dev = _device(dY)
    T, n_out = dY.shape
    n_in = Wq.shape[1]
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(Wq, "Wq", U8, (n_out, n_in), dev)
    _want(Ws, "Ws", U8, (n_out, n_in // 32), dev)
    if dX is None:
        dX = torch.empty((T, n_in), dtype=BF16, device=dev)
    _want(dX, "dX", BF16, (T, n_in), dev)
    need = sl_mxfp8_workspace_bytes(T, n_in, n_out)
    if workspace is None:
        workspace = wgrad_workspace(dev, need) if need else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("sl_linear_dgrad_mxfp8w", lib().sl_linear_dgrad_mxfp8w(
        _stream(dev), _ptr(dY), _ptr(Wq), _ptr(Ws), _ptr(dX), T, n_in, n_out, _ptr(workspace), nbytes))
    return dX


def sl_linear_wgrad_accum_mxfp8x(Xq, Xs, dY, main_grad, workspace=None):
    """main_grad += dY^T . deq(Xq, Xs) in fp32, in place."""
    dev = _device(Xq)
    T, n_in = Xq.shape
    n_out = dY.shape[1]
    _want(Xq, "Xq", U8, (T, n_in), dev)
    _want(Xs, "Xs", U8, (T, n_in // 32), dev)
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(main_grad, "main_grad", F32, (n_out, n_in), dev)
    need = sl_mxfp8_workspace_bytes(T, n_in, n_out)
    if workspace is None:
        workspace = wgrad_workspace(dev, need) if need else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("sl_linear_wgrad_accum_mxfp8x", lib().sl_linear_wgrad_accum_mxfp8x(
        _stream(dev), _ptr(Xq), _ptr(Xs), _ptr(dY), _ptr(main_grad), T, n_in, n_out, _ptr(workspace), nbytes))
    return main_grad


def sl_mxfp8_dequantize(q, s, out=None):
    """bf16 out[r, c] = E4M3(q[r, c]) * 2^(s[r, c/32] - 127) for codes q[R, C] and scales s[R, C/32]."""
    dev = _device(q)
    R, C = q.shape
    _want(q, "q", U8, (R, C), dev)
    _want(s, "s", U8, (R, C // 32), dev)
    if out is None:
        out = torch.empty((R, C), dtype=BF16, device=dev)
    _want(out, "out", BF16, (R, C), dev)
    check("sl_mxfp8_dequantize", lib().sl_mxfp8_dequantize(_stream(dev), _ptr(q), _ptr(s), _ptr(out), R, C))
    return out


# ---- all-MXFP8 step ---------------------------------------------------------------------------

def sl_mxfp8_quantize(x, rows=True, cols=True, out=None):
    """MX-quantise bf16 x[R, C]: returns (q_rows, s_rows, q_cols, s_cols); a copy not asked for is
    None.  Rowwise blocks run along C ([R, C] codes, [R, C/32] scales); columnwise blocks run down
    the columns and are stored transposed ([C, R] codes, [C, R/32] scales).  ``out`` may supply
    the four tensors."""
    dev = _device(x)
    R, C = x.shape
    _want(x, "x", BF16, (R, C), dev)
    if out is None:
        out = (torch.empty((R, C), dtype=U8, device=dev) if rows else None,
               torch.empty((R, C // 32), dtype=U8, device=dev) if rows else None,
               torch.empty((C, R), dtype=U8, device=dev) if cols else None,
               torch.empty((C, R // 32), dtype=U8, device=dev) if cols else None)
    qr, sr, qc, sc = out
    if qr is not None:
        _want(qr, "q_rows", U8, (R, C), dev)
        _want(sr, "s_rows", U8, (R, C // 32), dev)
    if qc is not None:
        _want(qc, "q_cols", U8, (C, R), dev)
        _want(sc, "s_cols", U8, (C, R // 32), dev)
    check("sl_mxfp8_quantize", lib().sl_mxfp8_quantize(
        _stream(dev), _ptr(x), R, C, _ptr(qr), _ptr(sr), _ptr(qc), _ptr(sc)))
    return qr, sr, qc, sc


def sl_linear_dgrad_mxfp8(dYq, dYs, WqT, WsT, dX=None):
    """dX[T,in] = deq(dYq, dYs)[T,out] . deq(WqT, WsT)[in,out]^T (bf16 out)."""
    dev = _device(dYq)
    T, n_out = dYq.shape
    n_in = WqT.shape[0]
    _want(dYq, "dYq", U8, (T, n_out), dev)
    _want(dYs, "dYs", U8, (T, n_out // 32), dev)
    _want(WqT, "WqT", U8, (n_in, n_out), dev)
    _want(WsT, "WsT", U8, (n_in, n_out // 32), dev)
    if dX is None:
        dX = torch.empty((T, n_in), dtype=BF16, device=dev)
    _want(dX, "dX", BF16, (T, n_in), dev)
    check("sl_linear_dgrad_mxfp8", lib().sl_linear_dgrad_mxfp8(
        _stream(dev), _ptr(dYq), _ptr(dYs), _ptr(WqT), _ptr(WsT), _ptr(dX), T, n_in, n_out))
    return dX


def sl_mxfp8_wgrad_workspace_bytes(T: int, n_in: int, n_out: int) -> int:
    return int(lib().sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out))


def sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, main_grad, workspace=None):
    """main_grad[out,in] += deq(dYqT, dYsT)[out,T] . deq(XqT, XsT)[in,T]^T in fp32, in place."""
    dev = _device(dYqT)
    n_out, T = dYqT.shape
    n_in = XqT.shape[0]
    _want(dYqT, "dYqT", U8, (n_out, T), dev)
    _want(dYsT, "dYsT", U8, (n_out, T // 32), dev)
    _want(XqT, "XqT", U8, (n_in, T), dev)
    _want(XsT, "XsT", U8, (n_in, T // 32), dev)
    _want(main_grad, "main_grad", F32, (n_out, n_in), dev)
    need = sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out)
    if workspace is None:
        workspace = wgrad_workspace(dev, need) if need else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("sl_linear_wgrad_accum_mxfp8", lib().sl_linear_wgrad_accum_mxfp8(
        _stream(dev), _ptr(dYqT), _ptr(dYsT), _ptr(XqT), _ptr(XsT), _ptr(main_grad), T, n_in, n_out,
        _ptr(workspace), nbytes))
    return main_grad


# ---- NVFP4 weights ------------------------------------------------------------------------------

def sl_nvfp4_materialize(Wq, Ws, Wm=None):
    """Wm[rows, cols] (bf16) = E2M1(Wq) * E4M3(Ws) per 16-element block, exactly; the tensor scale
    is not applied.  Wq [rows, cols/2] packed codes (element 2j in the low nibble of byte j),
    Ws [rows, cols/16] scale bytes."""
    dev = _device(Wq)
    rows, half = Wq.shape
    cols = 2 * half
    _want(Wq, "Wq", U8, (rows, half), dev)
    _want(Ws, "Ws", U8, (rows, cols // 16), dev)
    if Wm is None:
        Wm = torch.empty((rows, cols), dtype=BF16, device=dev)
    _want(Wm, "Wm", BF16, (rows, cols), dev)
    check("sl_nvfp4_materialize", lib().sl_nvfp4_materialize(
        _stream(dev), _ptr(Wq), _ptr(Ws), _ptr(Wm), rows, cols))
    return Wm


def sl_linear_fwd_nvfp4w(X, Wm, w_scale: float, Y=None):
    """Y[T,out] = w_scale * (X[T,in] . Wm[out,in]^T), scaled in fp32, rounded to bf16."""
    dev = _device(X)
    T, n_in = X.shape
    n_out = Wm.shape[0]
    _want(X, "X", BF16, (T, n_in), dev)
    _want(Wm, "Wm", BF16, (n_out, n_in), dev)
    if Y is None:
        Y = torch.empty((T, n_out), dtype=BF16, device=dev)
    _want(Y, "Y", BF16, (T, n_out), dev)
    check("sl_linear_fwd_nvfp4w", lib().sl_linear_fwd_nvfp4w(
        _stream(dev), _ptr(X), _ptr(Wm), float(w_scale), _ptr(Y), T, n_in, n_out))
    return Y


def sl_linear_dgrad_nvfp4w(dY, Wm, w_scale: float, dX=None):
    """dX[T,in] = w_scale * (dY[T,out] . Wm[out,in]), scaled in fp32, rounded to bf16."""
    dev = _device(dY)
    T, n_out = dY.shape
    n_in = Wm.shape[1]
    _want(dY, "dY", BF16, (T, n_out), dev)
    _want(Wm, "Wm", BF16, (n_out, n_in), dev)
    if dX is None:
        dX = torch.empty((T, n_in), dtype=BF16, device=dev)
    _want(dX, "dX", BF16, (T, n_in), dev)
    check("sl_linear_dgrad_nvfp4w", lib().sl_linear_dgrad_nvfp4w(
        _stream(dev), _ptr(dY), _ptr(Wm), float(w_scale), _ptr(dX), T, n_in, n_out))
    return dX
