"""Decoding of the storage formats the step consumes, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the upper 16 bits of an IEEE-754 binary32 value.
* E4M3FN (OCP 8-bit floating point, as used by MXFP8 per [GTP] section 1.3 "Low-precision
  gather"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  subnormals 2^-6 * m/8; the only NaN patterns are S.1111.111; no infinities.
* E8M0 (the MX shared scale): an unsigned biased exponent, value 2^(e-127); 0xFF is NaN.
* MX block size 32 along the contraction axis ([GTP] section 1.3, "Communication volume
  breakdown": one scale byte per 32 elements, 1/32 B per element).
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
