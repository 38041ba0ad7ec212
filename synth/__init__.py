"""Seeded synthetic inputs for the TP-sharded linear step.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side (tests, bench).
It draws random numbers and encodes them into the storage formats the step consumes; it holds
none of the step's own arithmetic (no products, no accumulation, no decoding for compute).

Storage formats produced:
  * bf16: numpy uint16 bit patterns, rounded from float32 draws with round-to-nearest-even.
  * MXFP8 (OCP Microscaling v1.0, E4M3 elements, E8M0 shared scale per 32-element block along
    the last axis): uint8 element codes plus uint8 biased scale exponents, one per block.

Seeding recipe: numpy Generator(PCG64(seed)) with
    seed = 1000*config + 100*param_index + 10*microbatch + role,    role: W=0, X=1, dY=2,
and weights always drawn with microbatch 0.  Weights are N(0, 0.02^2); activations and output
gradients are N(0, 1), following the workload descriptions of the Megatron-style runs (mock data,
random init) that the step is taken from.
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_X, ROLE_DY = 0, 1, 2
W_STD = 0.02

# E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; only S.1111.111 is NaN.
_E4M3_MAX = 448.0          # 1.75 * 2^8
_E4M3_EMAX = 8
_E4M3_EMIN = -6            # smallest normal exponent; subnormal spacing 2^-9
MX_BLOCK = 32


def seed_for(config: int, param_index: int, microbatch: int, role: int) -> int:
    """Seed of one tensor; weights (role 0) always use microbatch 0."""
    if role == ROLE_W:
        microbatch = 0
    return 1000 * config + 100 * param_index + 10 * microbatch + role


def normal_f32(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """float32 draws N(0, std^2) from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16 bit patterns.

    NaN inputs become a quiet NaN; finite values that round past the bf16 range become inf,
    as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def normal_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws stored as bf16 bit patterns (uint16)."""
    return f32_to_bf16_bits(normal_f32(shape, seed, std))


def _round_to_e4m3_grid(a: np.ndarray) -> np.ndarray:
    """Round non-negative float64 magnitudes to the E4M3FN value grid (RNE), saturating at 448."""
    out = np.zeros_like(a)
    nz = a > 0
    v = a[nz]
    e = np.floor(np.log2(v))
    e = np.maximum(e, _E4M3_EMIN)
    step = np.exp2(e - 3)                     # 3 mantissa bits
    r = np.rint(v / step) * step              # numpy rint rounds half to even
    out[nz] = np.minimum(r, _E4M3_MAX)
    return out


def _encode_e4m3(mag: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """Bit-encode grid magnitudes (exact E4M3 values) into uint8 codes."""
    code = np.zeros(mag.shape, dtype=np.uint8)
    nz = mag > 0
    v = mag[nz]
    e = np.floor(np.log2(v))
    sub = e < _E4M3_EMIN
    ef = np.where(sub, 0, e + 7).astype(np.int64)
    mant = np.where(sub, v / 2.0 ** -9, v / np.exp2(e) * 8 - 8)
    m = np.rint(mant).astype(np.int64)
    assert np.all(np.abs(mant - m) == 0), "magnitude not on the E4M3 grid"
    assert np.all((m >= 0) & (m <= 7)) and np.all(ef <= 15)
    code[nz] = (ef << 3 | m).astype(np.uint8)
    code[neg] |= np.uint8(0x80)
    return code


def mxfp8_quantize(x: np.ndarray):
    """Quantise float32 ``x`` (last axis a multiple of 32) to MXFP8 E4M3 with E8M0 block scales.

    Per 32-element block along the last axis (OCP MX v1.0 conversion):
      shared exponent X = floor(log2(amax)) - 8 (8 = largest E4M3 exponent), clamped to
      [-127, 127], stored biased by 127; an all-zero block stores 0 and zero codes;
      elements x / 2^X are rounded to nearest-even on the E4M3 grid, saturating at +-448.
    Returns (codes uint8 same shape as x, scales uint8 shape [..., K/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    k = x.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    xb = x.astype(np.float64).reshape(*x.shape[:-1], k // MX_BLOCK, MX_BLOCK)
    if not np.all(np.isfinite(xb)):
        raise ValueError("MXFP8 quantiser takes finite inputs only")
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - _E4M3_EMAX, -127)
    e = np.clip(e, -127, 127)
    scales = np.where(amax > 0, e + 127, 0).astype(np.uint8)
    scaled = xb / np.exp2(e)[..., None]
    mag = _round_to_e4m3_grid(np.abs(scaled))
    codes = _encode_e4m3(mag, np.signbit(scaled))
    return codes.reshape(x.shape), scales


def mxfp8_normal(shape, seed: int, std: float = 1.0):
    """N(0, std^2) float32 draws quantised to MXFP8 (codes, scales)."""
    return mxfp8_quantize(normal_f32(shape, seed, std))
