"""Seeded synthetic inputs for the TP-sharded linear step.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side (tests, bench).
It draws random numbers and encodes them into the storage formats the step consumes; it holds
none of the step's own arithmetic (no products, no accumulation, no decoding for compute).

Storage formats produced:
  * bf16: numpy uint16 bit patterns, rounded from float32 draws with round-to-nearest-even.
  * MXFP8 (OCP Microscaling v1.0, E4M3 elements, E8M0 shared scale per 32-element block along
    the last axis): uint8 element codes plus uint8 biased scale exponents, one per block.
  * NVFP4 (E2M1 elements packed two per byte, element 2j in the low nibble; one E4M3 scale per
    16-element block along the last axis; one fp32 per-tensor scale).

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


def mxfp8_quantize(x: np.ndarray):
    """Quantise float32 ``x`` (last axis a multiple of 32) to MXFP8 E4M3 with E8M0 block scales.

    Per 32-element block along the last axis (OCP MX v1.0 conversion):
      shared exponent X = floor(log2(amax)) - 8 (8 = largest E4M3 exponent), clamped to
      [-127, 127], stored biased by 127; an all-zero block stores 0 and zero codes;
      elements x / 2^X are rounded to nearest-even on the E4M3 grid, saturating at +-448.
    Returns (codes uint8 same shape as x, scales uint8 shape [..., K/32]).
    Works on float32 bit fields: floor(log2) of a normal float32 is its exponent field, and
    dividing by 2^X is exact for the inputs this module draws (no float32 subnormals arise).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = x.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("MXFP8 quantiser takes finite inputs only")
    xb = x.reshape(-1, k // MX_BLOCK, MX_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    if np.any((amax > 0) & (amax < np.float32(2.0 ** -126))):
        raise ValueError("float32 subnormal block maxima are not supported")
    e = (amax.view(np.int32) >> 23).astype(np.int32) - 127 - _E4M3_EMAX       # floor(log2 amax) - 8
    e = np.clip(e, -127, 127)
    zero_blk = amax == 0
    scales = np.where(zero_blk, 0, e + 127).astype(np.uint8)
    # multiply by 2^-X, built as an exact float32 power of two (X in [-127, 127] -> two factors)
    e1 = np.clip(-e, -126, 127)
    e2 = -e - e1
    f1 = ((e1 + 127).astype(np.int32) << 23).view(np.float32)
    f2 = ((e2 + 127).astype(np.int32) << 23).view(np.float32)
    v = xb * f1[..., None] * f2[..., None]
    a = np.abs(v)
    bits = a.view(np.uint32)
    # normals of E4M3 (a >= 2^-6): round the float32 mantissa to 3 bits, nearest-even
    rb = (bits + np.uint32(0x7FFFF) + ((bits >> np.uint32(20)) & np.uint32(1))) & np.uint32(0xFFF00000)
    rn = rb.view(np.float32)
    # subnormals of E4M3 (a < 2^-6): a fixed step 2^-9, nearest-even
    rs = np.rint(a * np.float32(512.0)) * np.float32(1.0 / 512.0)
    r = np.where(a < np.float32(2.0 ** -6), rs, rn)
    r = np.minimum(r, np.float32(_E4M3_MAX))
    rbits = r.view(np.uint32)
    ef = ((rbits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 127 + 7
    normal = r >= np.float32(2.0 ** -6)
    code_n = (np.clip(ef, 0, 15).astype(np.uint32) << np.uint32(3)) | ((rbits >> np.uint32(20)) & np.uint32(7))
    code_s = (r * np.float32(512.0)).astype(np.uint32)        # 0..8; 8 is the code of 2^-6
    code = np.where(normal, code_n, code_s).astype(np.uint8)
    code |= (np.signbit(v).astype(np.uint8) << np.uint8(7))
    code[zero_blk] = 0
    return code.reshape(x.shape), scales.reshape(*x.shape[:-1], k // MX_BLOCK)


def mxfp8_normal(shape, seed: int, std: float = 1.0):
    """N(0, std^2) float32 draws quantised to MXFP8 (codes, scales)."""
    return mxfp8_quantize(normal_f32(shape, seed, std))


# E2M1 magnitudes by code 0..7 (sign in bit 3)
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e4m3_rne_codes(v: np.ndarray) -> np.ndarray:
    """Non-negative float64 values -> E4M3 codes, round-to-nearest-even on the code grid,
    saturating at 448 (the grid is increasing in the code for codes 0x00..0x7E)."""
    grid = np.array([_e4m3_value(c) for c in range(0x7F)])
    v = np.minimum(v, 448.0)
    hi = np.clip(np.searchsorted(grid, v, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = np.abs(v - grid[lo]), np.abs(grid[hi] - v)
    return np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi))).astype(np.uint8)


def _e4m3_value(c: int) -> float:
    e, m = (c >> 3) & 0xF, c & 7
    return (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)


def nvfp4_quantize(x: np.ndarray):
    """Quantise float32 ``x`` [rows, cols] (cols a multiple of 16) to NVFP4 with NVIDIA's recipe:
    tensor scale t = amax / (6 * 448) (fp32); per 16-element block the E4M3 scale s = RNE(block
    amax / 6 / t); elements x / (s t) rounded to nearest-even on the E2M1 grid, saturating at 6.
    Returns (packed codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], t as a Python float).
    Works through 256-row chunks (large fresh arrays are slow to fault in).
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    amax = float(max(x.max(initial=0.0), -x.min(initial=0.0)))
    t = float(np.float32(amax / (6.0 * 448.0))) if amax > 0 else 1.0
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    svals = np.array([_e4m3_value(c) for c in range(0x7F)])
    for r0 in range(0, rows, 256):
        xb = x[r0:r0 + 256].astype(np.float64).reshape(-1, cols // 16, 16)
        bmax = np.abs(xb).max(axis=-1)
        sc = _e4m3_rne_codes(bmax / 6.0 / t)
        sval = svals[sc]
        with np.errstate(divide="ignore", invalid="ignore"):
            v = np.where(sval[..., None] > 0, np.abs(xb) / (sval[..., None] * t), 0.0)
        # nearest E2M1 magnitude index, ties to the even index: count the midpoints below v (a
        # midpoint whose upper neighbour has the even index counts when v reaches it)
        mag = np.zeros(v.shape, np.uint8)
        for mid, upper_even in ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
                                (2.5, False), (3.5, True), (5.0, False)):
            mag += (v >= mid) if upper_even else (v > mid)
        codes = (mag | ((np.signbit(xb) & (mag > 0)).astype(np.uint8) << 3)).reshape(-1, cols)
        packed[r0:r0 + 256] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        scales[r0:r0 + 256] = sc
    return packed, scales, t


def nvfp4_normal(shape, seed: int, std: float = 1.0):
    """N(0, std^2) float32 draws quantised to NVFP4 (packed codes, scales, tensor scale)."""
    return nvfp4_quantize(normal_f32(shape, seed, std))
