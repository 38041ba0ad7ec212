"""Decoding of the storage formats the step consumes, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.
* E4M3FN (OCP 8-bit floating point, as used by MXFP8 per [GTP] section 1.3 "Low-precision
  gather"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals 2^-6 * m/8; the only NaN patterns are S.1111.111; no infinities.
* E8M0 (the MX shared scale): an unsigned biased exponent, value 2^(e-127); 0xFF is NaN.
* MX block size 32 along the contraction axis ([GTP] section 1.3, "Communication volume
  breakdown": one scale byte per 32 elements, 1/32 B per element).
* E2M1 (the NVFP4 element, [GTP] section 1.3 "Native NVFP4 param": packed 4-bit kFloat4E2M1):
  sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent field 0 encodes the subnormal
  0.5 * m; values 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte, element 2j in the low nibble.
* NVFP4 ([GTP] section 1.3 table: block 16, 0.5 + 1/16 bytes per element, per-tensor scale set at
  the optimizer-step quantize): deq = E2M1(code) * E4M3(block scale) * tensor scale (fp32); the
  scale encodings are NVIDIA's NVFP4 definition, which the pages name but do not spell out.
* MX quantisation (the pages fix only the block of 32 and per-block scaling with no tensor-wide
  amax, [GTP] section 1.3; the rule below is the OCP Microscaling v1.0 conversion): per block,
  shared exponent X = floor(log2 amax) - 8 (8 = the largest E4M3 exponent) clamped to
  [-127, 127] and stored biased by 127; each element x / 2^X rounded to the nearest E4M3 value,
  ties to the even code, saturating at +-448; the sign of x is kept (a negative element that
  rounds to zero is -0); an all-zero block stores scale 0 and zero codes.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code by the textbook definition (scalar, for tables and pins)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN codes (uint8 array) to float64 through the 256-entry definition table."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_to_f64(s: np.ndarray) -> np.ndarray:
    """Decode E8M0 biased exponents to float64 powers of two (0xFF -> NaN)."""
    s = np.asarray(s, dtype=np.uint8).astype(np.float64)
    v = np.exp2(s - 127.0)
    return np.where(s == 255.0, np.nan, v)


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """deq(q, s) = E4M3(q) * 2^(s - 127), one scale per ``block`` elements of the last axis."""
    codes = np.asarray(codes, dtype=np.uint8)
    k = codes.shape[-1]
    assert k % block == 0 and scales.shape[-1] == k // block
    v = e4m3_to_f64(codes).reshape(*codes.shape[:-1], k // block, block)
    return (v * e8m0_to_f64(scales)[..., None]).reshape(codes.shape)


_NONNEG_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: 0 .. 448, increasing


def _e4m3_encode_nonneg(r: np.ndarray) -> np.ndarray:
    """Code of non-negative E4M3 values (exact grid points), through the inverse of the table."""
    grid = E4M3_TABLE[:0x7F]
    idx = np.searchsorted(grid, r)
    assert np.all(grid[idx] == r), "not an E4M3 grid point"
    return _NONNEG_CODES[idx]


def mx_quantize(x: np.ndarray, block: int = 32):
    """MX-quantise real ``x`` along its last axis into (E4M3 codes, E8M0 scales), in float64.

    Follows the OCP MX v1.0 conversion stated in the module docstring, step by step:
    floor(log2 amax) comes from frexp (amax = m 2^E, m in [0.5, 1) -> E - 1), the division by
    2^X is exact in float64, and rounding to the E4M3 grid uses the grid spacing of the value's
    binade (2^(e-3) for normals, 2^-9 below 2^-6) with numpy's round-half-even.
    """
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    assert k % block == 0 and np.all(np.isfinite(x))
    xb = x.reshape(-1, k // block, block)
    amax = np.abs(xb).max(axis=-1)
    zero = amax == 0
    _, E = np.frexp(np.where(zero, 1.0, amax))
    X = np.clip(E - 1 - 8, -127, 127)
    v = xb / np.exp2(X)[..., None]
    a = np.abs(v)
    _, ea = np.frexp(np.where(a == 0, 1.0, a))
    q = np.where(a >= 2.0 ** -6, np.exp2(ea - 1 - 3), 2.0 ** -9)       # grid spacing at a
    r = np.minimum(np.rint(a / q) * q, 448.0)
    codes = _e4m3_encode_nonneg(r) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    codes[np.broadcast_to(zero[..., None], codes.shape)] = 0
    scales = np.where(zero, 0, X + 127).astype(np.uint8)
    return codes.reshape(x.shape).astype(np.uint8), scales.reshape(*x.shape[:-1], k // block)


def mx_quantize_cols(x: np.ndarray, block: int = 32):
    """Columnwise MX quantisation of a 2-D ``x`` [R, C]: blocks of 32 run down the columns and the
    result is stored transposed, codes [C, R] and scales [C, R/32] -- the layout in which a GEMM
    contracting over R reads it with k contiguous."""
    return mx_quantize(np.asarray(x, dtype=np.float64).T, block)


def e2m1_value(code: int) -> float:
    """Value of one E2M1 code by the definition (scalar, for tables and pins)."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 0x3, code & 0x1
    if e == 0:
        return sign * 0.5 * m
    return sign * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def nvfp4_dequant(packed: np.ndarray, scales: np.ndarray, tensor_scale: float, block: int = 16) -> np.ndarray:
    """deq = E2M1(code) * E4M3(scale) * tensor_scale for packed codes [rows, cols/2] (element 2j in
    the low nibble of byte j) and E4M3 block scales [rows, cols/16]."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    v = E2M1_TABLE[codes].reshape(rows, -1, block)
    sc = e4m3_to_f64(scales)
    assert sc.shape == (rows, 2 * half // block)
    return (v * sc[..., None]).reshape(rows, 2 * half) * float(np.float32(tensor_scale))
