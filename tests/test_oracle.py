"""Pins of the oracle against facts fixed outside the oracle itself.

Each test names what it pins: values the pages print, closed forms, hand-computed examples,
brute force on tiny shapes, algebraic invariants of the TP decomposition, and the format tables.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import layout, linear, numerics, shapes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# Storage-format decoders
# ---------------------------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    # IEEE binary32 upper halves: 1.0, -2.0, +inf, smallest subnormal, largest finite, 0.5
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x7F7F, 0x3F00], dtype=np.uint16)
    v = numerics.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and np.isinf(v[2])
    assert v[3] == 2.0 ** -133
    assert v[4] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert v[5] == 0.5


def test_e4m3_table_closed_form_values():
    t = numerics.E4M3_TABLE
    # OCP 8-bit FP spec, E4M3: bias 7, max normal 448 (S.1111.110), min normal 2^-6,
    # min subnormal 2^-9, NaN only at S.1111.111, no infinities.
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) == -1
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0 and t[0x30] == 0.5 and t[0x40] == 2.0
    assert t[0x77] == 240.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254 and not np.isinf(t).any()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])


def test_e8m0_decode():
    s = np.array([0, 1, 127, 128, 254, 255], dtype=np.uint8)
    v = numerics.e8m0_to_f64(s)
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 1.0 and v[3] == 2.0
    assert v[4] == 2.0 ** 127 and np.isnan(v[5])


def test_mxfp8_dequant_unit_and_uniform_scales():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                   # avoid NaN codes
    unit = numerics.mxfp8_dequant(codes, np.full((3, 2), 127, np.uint8))
    assert np.array_equal(unit, numerics.E4M3_TABLE[codes])
    sc = np.array([[120, 130]] * 3, dtype=np.uint8)
    d = numerics.mxfp8_dequant(codes, sc)
    assert np.array_equal(d[:, :32], unit[:, :32] * 2.0 ** -7)
    assert np.array_equal(d[:, 32:], unit[:, 32:] * 2.0 ** 3)


def test_quantiser_round_trip_powers_of_two_exact():
    # blocks whose elements are powers of two within 2^-9 of the block max are exact in E4M3
    x = np.array([[2.0 ** (-(i % 9)) * (-1) ** i for i in range(32)],
                  [0.0] * 32], dtype=np.float32)
    q, s = synth.mxfp8_quantize(x)
    assert s[1, 0] == 0 and not q[1].any()                 # all-zero block
    back = numerics.mxfp8_dequant(q, s)
    assert np.array_equal(back, x.astype(np.float64))


def test_quantiser_error_bound():
    # RNE to 3 mantissa bits: |x - deq| <= 2^-4 |x| on normals, <= half subnormal step otherwise;
    # with X = floor(log2 amax) - 8 a block max scales into [256, 512), and magnitudes above 448
    # saturate to 448 (OCP MX conversion), so there the error is |x| - 448 * 2^X.
    x = synth.normal_f32((64, 256), seed=7)
    q, s = synth.mxfp8_quantize(x)
    back = numerics.mxfp8_dequant(q, s)
    scale = numerics.e8m0_to_f64(s).repeat(32, axis=-1)
    err = np.abs(back - x)
    sat = np.abs(x) > 448 * scale
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10)
    bound = np.where(sat, np.abs(x) - 448 * scale, bound)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.all(np.abs(back[sat]) == 448 * scale[sat])
    # block maxima land near the top of the E4M3 range (floor(log2 amax) - 8 keeps amax < 512*2^X)
    assert np.all(np.abs(back).reshape(64, 8, 32).max(-1) <= 448 * numerics.e8m0_to_f64(s))


def test_bf16_rounding_of_inputs_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: RNE goes to the even mantissa (1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20], np.float32)
    v = numerics.bf16_bits_to_f64(synth.f32_to_bf16_bits(x))
    assert v[0] == 1.0 and v[1] == 1 + 2 ** -6 and v[2] == -1.0 and v[3] == 1 + 2 ** -7


# ---------------------------------------------------------------------------------------------
# GEMM formulas
# ---------------------------------------------------------------------------------------------

def test_hand_computed_2x3():
    # A non-symmetric, non-square example worked by hand: catches transposed operands.
    X = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])          # [T=2, in=3]
    W = np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.0]])        # [out=2, in=3]
    dY = np.array([[1.0, -1.0], [0.5, 2.0]])                 # [T=2, out=2]
    assert np.array_equal(linear.linear_fwd(X, W), [[-2.0, 4.0], [-2.0, 13.0]])
    assert np.array_equal(linear.linear_dgrad(dY, W), [[-1.0, -1.0, -1.0], [4.5, 2.0, -0.5]])
    G0 = np.array([[10.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    # dY^T X = [[1*1+0.5*4, 1*2+0.5*5, 1*3+0.5*6], [-1*1+2*4, -1*2+2*5, -1*3+2*6]]
    want = G0 + np.array([[3.0, 4.5, 6.0], [7.0, 8.0, 9.0]])
    assert np.array_equal(linear.linear_wgrad_accum(G0, X, dY), want)


@pytest.mark.parametrize("T,n_in,n_out", [(1, 1, 1), (2, 3, 5), (5, 17, 3), (3, 2, 33), (17, 5, 2)])
def test_brute_force_tiny(T, n_in, n_out):
    rng = np.random.default_rng(T * 100 + n_in * 10 + n_out)
    X = synth.f32_to_bf16_bits(rng.standard_normal((T, n_in)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.standard_normal((n_out, n_in)).astype(np.float32))
    dY = synth.f32_to_bf16_bits(rng.standard_normal((T, n_out)).astype(np.float32))
    G0 = rng.standard_normal((n_out, n_in))
    tol = 1e-12
    np.testing.assert_allclose(linear.linear_fwd(X, W), linear.fwd_brute(X, W), rtol=tol, atol=tol)
    np.testing.assert_allclose(linear.linear_dgrad(dY, W), linear.dgrad_brute(dY, W), rtol=tol, atol=tol)
    np.testing.assert_allclose(linear.linear_wgrad_accum(G0, X, dY),
                               linear.wgrad_accum_brute(G0, X, dY), rtol=tol, atol=tol)


def test_exact_special_cases():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((7, 5))
    X = np.zeros((4, 5)); X[np.arange(4), [0, 2, 4, 1]] = 1.0     # one-hot rows
    Y = linear.linear_fwd(X, W)
    for t, i0 in enumerate([0, 2, 4, 1]):
        assert np.array_equal(Y[t], W[:, i0])                     # a column of W
    dY = np.zeros((3, 7)); dY[np.arange(3), [6, 0, 3]] = 1.0
    dX = linear.linear_dgrad(dY, W)
    for t, o0 in enumerate([6, 0, 3]):
        assert np.array_equal(dX[t], W[o0])                       # a row of W
    Wsq = np.eye(5)
    X2 = rng.standard_normal((6, 5))
    assert np.array_equal(linear.linear_fwd(X2, Wsq), X2)          # W = I
    x1 = rng.standard_normal((1, 5)); g1 = rng.standard_normal((1, 7))
    assert np.array_equal(linear.linear_wgrad_accum(np.zeros((7, 5)), x1, g1), np.outer(g1[0], x1[0]))


def test_non_finite_inputs_propagate_as_the_definition_says():
    """The oracle's products on NaN / inf inputs agree with the brute-force loops entry by entry
    (NaN where a NaN term or +inf and -inf terms meet, +-inf where only infinite terms of one sign
    do), so it can serve as the reference for non-finite propagation."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal((5, 6)); W = rng.standard_normal((4, 6)); dY = rng.standard_normal((5, 4))
    G0 = rng.standard_normal((4, 6))
    X[1, 2] = np.nan; X[3, 4] = np.inf; dY[0, 1] = -np.inf; dY[2, 3] = np.nan; G0[2, 5] = np.inf
    with np.errstate(invalid="ignore"):
        pairs = [(linear.linear_fwd(X, W), linear.fwd_brute(X, W)),
                 (linear.linear_dgrad(dY, W), linear.dgrad_brute(dY, W)),
                 (linear.linear_wgrad_accum(G0, X, dY), linear.wgrad_accum_brute(G0, X, dY))]
    for got, want in pairs:
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(np.isinf(got), np.isinf(want))
        inf = np.isinf(want)
        assert np.array_equal(np.sign(got[inf]), np.sign(want[inf]))
        fin = np.isfinite(want)
        np.testing.assert_allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12)
    assert np.isnan(pairs[0][0][1]).all() and np.isnan(pairs[2][0][:, 2]).all()


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(4)
    X, W, dY = rng.standard_normal((9, 6)), rng.standard_normal((4, 6)), rng.standard_normal((9, 4))
    assert np.array_equal(linear.linear_fwd(X * 8, W / 4), linear.linear_fwd(X, W) * 2)
    assert np.array_equal(linear.linear_dgrad(dY / 2, W * 16), linear.linear_dgrad(dY, W) * 8)
    z = np.zeros((4, 6))
    assert np.array_equal(linear.linear_wgrad_accum(z, X * 4, dY * 4), linear.linear_wgrad_accum(z, X, dY) * 16)


# ---------------------------------------------------------------------------------------------
# Accumulation ([ATLAS-TP] section 4.2 fusion; [ATLAS-BUF] sections 6.4 and 6.6)
# ---------------------------------------------------------------------------------------------

def test_accumulation_linearity_and_zero_start():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((6, 4))
    Xs = [rng.standard_normal((8, 4)) for _ in range(3)]
    dYs = [rng.standard_normal((8, 6)) for _ in range(3)]
    _, _, G = linear.step(W, Xs, dYs)
    parts = sum(dY.T @ X for X, dY in zip(Xs, dYs))
    np.testing.assert_allclose(G, parts, rtol=1e-12, atol=1e-12)
    # the sum of micro-batch wgrads equals one wgrad over the concatenated tokens
    np.testing.assert_allclose(G, linear.linear_wgrad(np.vstack(Xs), np.vstack(dYs)), rtol=1e-12, atol=1e-12)
    _, _, G1 = linear.step(W, Xs[:1], dYs[:1])
    assert np.array_equal(G1, linear.linear_wgrad(Xs[0], dYs[0]))
    _, _, G2 = linear.step(W, [Xs[0]] * 2, [dYs[0]] * 2)
    assert np.array_equal(G2, 2 * G1)                                  # same data twice, bitwise
    _, _, Gc = linear.step(W, Xs[1:], dYs[1:], main_grad0=G1)          # accumulation continues
    np.testing.assert_allclose(Gc, G, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# TP sharding invariants ([ATLAS-TP] section 1: column then row needs one reduction per pair)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("tp", [1, 2, 4])
def test_column_then_row_composition(tp):
    rng = np.random.default_rng(10 + tp)
    h, f, T = 8, 16, 5
    W1 = rng.standard_normal((f, h))        # column-parallel: split along out (rows)
    W2 = rng.standard_normal((h, f))        # row-parallel: split along in (columns)
    X = rng.standard_normal((T, h))
    dY = rng.standard_normal((T, h))
    full_Z = linear.linear_fwd(X, W1)
    full_Y = linear.linear_fwd(full_Z, W2)
    c = f // tp
    shards = [(W1[r * c:(r + 1) * c], W2[:, r * c:(r + 1) * c]) for r in range(tp)]
    # forward: each rank's column output feeds its row shard; partial sums add to the full Y
    partial = [linear.linear_fwd(linear.linear_fwd(X, a), b) for a, b in shards]
    np.testing.assert_allclose(sum(partial), full_Y, rtol=1e-12, atol=1e-12)
    # backward (identity activation): row dgrad is the full dZ restricted to the rank's slice
    full_dZ = linear.linear_dgrad(dY, W2)
    for r, (a, b) in enumerate(shards):
        np.testing.assert_allclose(linear.linear_dgrad(dY, b), full_dZ[:, r * c:(r + 1) * c], rtol=1e-12, atol=1e-12)
    # column dgrad partials summed over ranks give the unsharded dX (the all-reduce of f)
    dX_parts = [linear.linear_dgrad(full_dZ[:, r * c:(r + 1) * c], a) for r, (a, _) in enumerate(shards)]
    np.testing.assert_allclose(sum(dX_parts), linear.linear_dgrad(full_dZ, W1), rtol=1e-12, atol=1e-12)
    # each shard's wgrad is the matching slice of the unsharded wgrad
    G1 = linear.linear_wgrad(X, full_dZ)
    G2 = linear.linear_wgrad(full_Z, dY)
    for r, (a, b) in enumerate(shards):
        zr = linear.linear_fwd(X, a)
        np.testing.assert_allclose(linear.linear_wgrad(X, full_dZ[:, r * c:(r + 1) * c]), G1[r * c:(r + 1) * c], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(linear.linear_wgrad(zr, dY), G2[:, r * c:(r + 1) * c], rtol=1e-12, atol=1e-12)


def test_tp1_shard_is_the_unsharded_layer():
    rng = np.random.default_rng(20)
    W = rng.standard_normal((6, 4)); X = rng.standard_normal((3, 4)); dY = rng.standard_normal((3, 6))
    shard = W[0:6, 0:4]                                   # the only shard at TP=1
    assert np.array_equal(linear.linear_fwd(X, shard), linear.linear_fwd(X, W))
    assert np.array_equal(linear.linear_dgrad(dY, shard), linear.linear_dgrad(dY, W))


# ---------------------------------------------------------------------------------------------
# Shapes ([MEGA-SRC] section 1)
# ---------------------------------------------------------------------------------------------

def test_llama_1b_param_ledger():
    cfg = shapes.LLAMA_1B
    assert shapes.per_layer_params(**cfg) == 60_821_504
    assert cfg["L"] * shapes.per_layer_params(**cfg) == 973_144_064
    assert cfg["v"] * cfg["h"] == 262_668_288
    assert shapes.total_params(**cfg) == 1_498_482_688
    per_card = shapes.total_params(**cfg) / (2 * 2)       # PP=2 stages, TP=2 halves
    assert round(per_card / 1e6, 1) == 374.6
    assert round(per_card * (2 + 4 + 12 / 2) / 1e9, 2) == 4.50   # 12 B per TP-local param
    assert round(per_card * 12 / 2 ** 30, 2) == 4.19


def test_tp2_shards_add_up_to_the_layer():
    cfg = shapes.LLAMA_1B
    sh = shapes.tp_shard_shapes(**cfg, tp=2)
    assert sh == {"linear_qkv": (1536, 2048), "linear_proj": (2048, 1024),
                  "linear_fc1": (8192, 2048), "linear_fc2": (2048, 4096)}
    per_rank = sum(o * i for o, i in sh.values())
    assert per_rank == 30_408_704
    assert 2 * per_rank + 2 * cfg["h"] == shapes.per_layer_params(**cfg)


# ---------------------------------------------------------------------------------------------
# Layout ([ATLAS-BUF] sections 4-5, [MEGA-SRC] section 6.3 toy)
# ---------------------------------------------------------------------------------------------

def test_toy_layout_matches_printed_output():
    g = json.load(open(os.path.join(GOLDEN, "toy_layout.json")))
    names = [n for n, _ in g["definition_order"]]
    lay = layout.build_layout([k for _, k in g["definition_order"]], param_align=g["param_align"],
                              bucket_size=None, dp=g["dp"], divisor=g["divisor"])
    exp = g["expected"]
    assert lay.numel == exp["numel"]
    assert lay.buckets[0][1] - lay.buckets[0][2] == exp["pad"]
    for i, n in enumerate(names):
        assert [lay.start[i], lay.end[i]] == exp["ranges"][n]
    shards = layout.shard_ranges(0, lay.numel, g["dp"])
    assert shards[0][1] == exp["shard_boundary"]
    wl = names.index("WL")
    lo, hi = lay.start[wl], lay.end[wl]
    assert [lo - lo, min(hi, shards[0][1]) - 1 - lo] == exp["WL_elements_on_rank0"]
    assert [shards[1][0] - lo, hi - 1 - lo] == exp["WL_elements_on_rank1"]


def test_7b_bucket_ledger():
    # [ATLAS-BUF] section 8: P' = 1.875e9 elements per rank, dp=64, bucket_size = max(40M, 64M)
    # = 64M elements -> about 29 full buckets + 1 tail, padding <= 2^16 - 1 per bucket (high
    # bus-bandwidth padding), about 1.9M padding elements in total.  Parameters of 1e6 elements
    # (a multiple of 64, so no start padding) stand in for the fine-grained parameter list.
    dp = 64
    bs = layout.default_bucket_size(dp)
    assert bs == 64_000_000
    lay = layout.build_layout([1_000_000] * 1875, param_align=64, bucket_size=bs, dp=dp,
                              divisor=layout.bucket_divisor(dp, high_busbw=True))
    full = [b for b in lay.buckets if b[2] >= bs]
    assert len(full) == 29 and len(lay.buckets) == 30
    pads = [b[1] - b[2] for b in lay.buckets]
    assert max(pads) <= 2 ** 16 - 1 and all(b[1] % dp == 0 for b in lay.buckets)
    assert sum(pads[:29]) <= 29 * (2 ** 16 - 1)
    assert round(lay.numel * 4 / 1e9, 1) == 7.5                       # grad_data fp32 7.5 GB
    assert round(lay.numel * 2 / 1e9, 2) == 3.75                      # param_data bf16 3.75 GB
    assert round(bs * 4 / 1e6) == 256                                 # 256 MB per bucket RS


def test_divisor_and_default_bucket_size():
    assert layout.bucket_divisor(1) == 128 and layout.bucket_divisor(2) == 128
    assert layout.bucket_divisor(3) == 384 and layout.bucket_divisor(64) == 128
    assert layout.bucket_divisor(64, high_busbw=True) == 65536
    assert layout.bucket_divisor(3, high_busbw=True) == 3 * 65536
    assert layout.default_bucket_size(1) == 40_000_000
    assert layout.default_bucket_size(64) == 64_000_000


def test_config_layouts():
    # C2, one TP=2 rank's MLP: fc1 [8192,2048] then fc2 [2048,4096] in definition order.
    lay = layout.build_layout([8192 * 2048, 2048 * 4096], bucket_size=layout.default_bucket_size(1))
    assert (lay.start, lay.end) == ([8_388_608, 0], [25_165_824, 8_388_608])
    assert lay.numel == 25_165_824 and len(lay.buckets) == 1
    # C4, 7B-class layer shards at dp=1 (qkv, proj, fc1, fc2): bucket 0 closes after fc1.
    n = [6144 * 4096, 4096 * 2048, 11008 * 4096, 4096 * 5504]
    lay = layout.build_layout(n, bucket_size=layout.default_bucket_size(1))
    assert lay.start == [76_021_760, 67_633_152, 22_544_384, 0]
    assert lay.bucket_id == [1, 1, 0, 0]
    assert lay.buckets == [(0, 67_633_152, 67_633_152), (67_633_152, 33_554_432, 33_554_432)]
    # C1: a single [512,256] weight at offset 0 of a 131072-element buffer (a multiple of 64)
    lay = layout.build_layout([512 * 256], bucket_size=None)
    assert (lay.start, lay.numel) == ([0], 131_072) and lay.numel % 64 == 0


@pytest.mark.parametrize("seed", range(6))
def test_layout_properties_random(seed):
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(1, 5000, size=int(rng.integers(1, 40)))]
    dp = int(rng.choice([1, 2, 3, 8]))
    bs = int(rng.integers(100, 20000))
    div = layout.bucket_divisor(dp)
    lay = layout.build_layout(numels, param_align=64, bucket_size=bs, dp=dp, divisor=div)
    n = len(numels)
    for i in range(n):
        assert lay.start[i] % 64 == 0 and lay.end[i] - lay.start[i] == numels[i]
    for i in range(n - 1):          # reverse order: a later-defined param sits at a lower offset
        assert lay.end[i + 1] <= lay.start[i]
    prev = 0
    for b, (off, num, unp) in enumerate(lay.buckets):
        assert off == prev and num % div == 0 and num - unp < div and unp <= num
        members = [i for i in range(n) if lay.bucket_id[i] == b]
        assert members, "no empty buckets"
        last = min(members)          # the bucket's last-placed param (lowest definition index)
        assert lay.end[last] - off == unp
        if b < len(lay.buckets) - 1:
            assert unp >= bs          # a bucket closes only once it reaches bucket_size ...
            before = [lay.end[i] for i in members if i != last]
            assert all(e - off < bs for e in before)   # ... and not earlier
        prev = off + num
    assert lay.numel == prev


def _scalar_e4m3_quant(block):
    """One block by the OCP MX rule, element by element in Python floats (test reference)."""
    amax = max(abs(float(v)) for v in block)
    if amax == 0:
        return [0] * len(block), 0
    X = min(max(math.floor(math.log2(amax)) - 8, -127), 127)
    grid = sorted({numerics.e4m3_value(c) for c in range(0x7F)})          # non-negative values
    codes = []
    for v in block:
        a = abs(float(v)) / 2.0 ** X
        if a >= 448:
            r = 448.0
        else:
            hi = next(g for g in grid if g >= a)
            lo = max(g for g in grid if g <= a)
            if hi - a < a - lo:
                r = hi
            elif a - lo < hi - a:
                r = lo
            else:                                                           # tie: even code
                cl, ch = grid.index(lo), grid.index(hi)
                r = lo if cl % 2 == 0 else hi
        c = grid.index(r) | (0x80 if math.copysign(1, float(v)) < 0 else 0)
        codes.append(c)
    return codes, X + 127


def test_quantiser_matches_scalar_rule():
    rng = np.random.default_rng(8)
    blocks = [rng.standard_normal(32).astype(np.float32) * np.float32(s) for s in (1, 0.02, 3e-3, 7e4)]
    tie = np.array([1.0, 1.0625, 1.1875, 0.25 + 2 ** -11, 2 ** -14, 2 ** -16 * 3] + [0.5] * 26, np.float32)
    blocks += [tie, -tie, np.full(32, 460.0, np.float32), np.zeros(32, np.float32)]
    x = np.stack(blocks)
    q, s = synth.mxfp8_quantize(x)
    for b in range(x.shape[0]):
        codes, sc = _scalar_e4m3_quant(x[b])
        assert s[b, 0] == sc and list(q[b]) == codes, b


# ---- the oracle's own MX quantiser (the quantisation step of the MXFP8 backward path) ----------

def test_oracle_quantiser_matches_scalar_rule():
    """numerics.mx_quantize against the element-by-element nearest-grid search above, on normal
    draws of several magnitudes, exact ties, saturating values, zeros and signed zeros."""
    rng = np.random.default_rng(18)
    blocks = [rng.standard_normal(32) * s for s in (1, 0.02, 3e-3, 7e4, 1e-30)]
    tie = np.array([1.0, 1.0625, 1.1875, 0.25 + 2 ** -11, 2 ** -14, 2 ** -16 * 3] + [0.5] * 26)
    signed_zero = np.array([-0.0, 0.0, 3.0] + [-2.0 ** -12] * 29)
    blocks += [tie, -tie, np.full(32, 460.0), np.zeros(32), signed_zero]
    x = np.stack(blocks)
    q, s = numerics.mx_quantize(x)
    for b in range(x.shape[0]):
        codes, sc = _scalar_e4m3_quant(x[b])
        assert s[b, 0] == sc and list(q[b]) == codes, b


def test_oracle_quantiser_every_bf16_below_the_block_max():
    """Every positive finite bf16 magnitude up to 256, each in a block whose maximum is 256
    (shared exponent 0): the code is the nearest E4M3 value, ties to even, by brute force."""
    bits = np.arange(1, 0x4380 + 1, dtype=np.uint32)                   # bf16 0x0001 .. 256.0
    vals = (bits << 16).view(np.float32).astype(np.float64)
    vals = vals[vals <= 256.0]
    n = (vals.size + 30) // 31
    x = np.full((n, 32), 0.0)
    x[:, 31] = 256.0
    x[:, :31].flat[: vals.size] = vals
    q, s = numerics.mx_quantize(x)
    assert np.all(s == 127)
    grid = np.array(sorted({numerics.e4m3_value(c) for c in range(0x7F)}))
    codes = np.array(sorted(range(0x7F), key=numerics.e4m3_value))
    got = q[:, :31].flat[: vals.size]
    lo = np.searchsorted(grid, vals, side="right") - 1
    hi = np.minimum(lo + 1, grid.size - 1)
    dlo, dhi = vals - grid[lo], grid[hi] - vals
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    assert np.array_equal(got, codes[pick])


def test_oracle_quantiser_scale_range_and_bound():
    """amax / 2^X lies in [256, 512) for unclamped blocks; |x - deq| is at most half a grid step
    (2^(e-4) for an element of binade 2^e after scaling) below the saturation point."""
    rng = np.random.default_rng(19)
    x = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    q, s = numerics.mx_quantize(x)
    X = s.astype(np.int64) - 127
    amax = np.abs(x.reshape(64, 4, 32)).max(-1)
    ratio = amax / np.exp2(X)
    assert np.all((ratio >= 256) & (ratio < 512))
    back = numerics.mxfp8_dequant(q, s)
    v = np.abs(x.reshape(64, 4, 32)) / np.exp2(X)[..., None]
    step = np.where(v >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3), 2.0 ** -9)
    err = np.abs(x - back).reshape(64, 4, 32) / np.exp2(X)[..., None]
    ok = (v > 448) | (err <= step / 2 + 1e-300)
    assert np.all(ok)


def test_columnwise_quantisation_blocks_run_down_columns():
    """A column whose 32-row blocks are power-of-two multiples of E4M3 values round-trips exactly
    through the transposed columnwise copy.  (Codes with mantissa 7 are left out: a block maximum
    of 1.875 * 2^e scales to 480 and saturates to 448 under the shared-exponent rule.)"""
    rng = np.random.default_rng(20)
    codes = rng.integers(0, 0x7F, (64, 96)).astype(np.uint8)
    codes[(codes & 7) == 7] -= 1
    x = numerics.e4m3_to_f64(codes) * np.exp2(rng.integers(-10, 10, (1, 96)))
    q, s = numerics.mx_quantize_cols(x)
    assert q.shape == (96, 64) and s.shape == (96, 2)
    back = numerics.mxfp8_dequant(q, s)
    assert np.array_equal(back, x.T)


@pytest.mark.parametrize("T,n_in,n_out", [(32, 32, 32), (64, 96, 32), (96, 32, 64)])
def test_mxfp8_backward_products_brute_force(T, n_in, n_out):
    """dgrad and wgrad over both-MXFP8 operands equal the triple loops over the dequantised
    values, with the weight and the gradients in the layouts the kernels read."""
    rng = np.random.default_rng(T + n_in + n_out)
    dY = rng.standard_normal((T, n_out))
    W = rng.standard_normal((n_out, n_in)) * 0.02
    X = rng.standard_normal((T, n_in))
    G0 = rng.standard_normal((n_out, n_in))
    dYq, dYs = numerics.mx_quantize(dY)
    WqT, WsT = numerics.mx_quantize_cols(W)
    dYqT, dYsT = numerics.mx_quantize_cols(dY)
    XqT, XsT = numerics.mx_quantize_cols(X)
    dX = linear.linear_dgrad_mxfp8(dYq, dYs, WqT, WsT)
    want = linear.dgrad_brute(numerics.mxfp8_dequant(dYq, dYs), numerics.mxfp8_dequant(WqT, WsT).T)
    assert np.allclose(dX, want, rtol=1e-12, atol=1e-12)
    G = linear.linear_wgrad_accum_mxfp8(G0, dYqT, dYsT, XqT, XsT)
    want = linear.wgrad_accum_brute(G0, numerics.mxfp8_dequant(XqT, XsT).T, numerics.mxfp8_dequant(dYqT, dYsT).T)
    assert np.allclose(G, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# NVFP4 weights: E2M1 elements, E4M3 scales per 16 elements, one fp32 tensor scale
# ---------------------------------------------------------------------------------------------

def test_e2m1_table_values():
    # OCP MX v1.0 FP4 E2M1: bias 1, max normal 6 (0.111), min normal 1, one subnormal 0.5;
    # no infinities or NaN; the 16 codes give 15 distinct values (+0 and -0).
    t = numerics.E2M1_TABLE
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(t[8:], -t[:8]) and math.copysign(1, t[8]) == -1
    assert np.all(np.isfinite(t))


def test_nvfp4_dequant_hand_worked_bytes():
    """Two rows of 32 elements with hand-decoded bytes: nibble order (element 2j low), scale per
    16-element block, E4M3 scale decode and the tensor scale."""
    packed = np.zeros((2, 16), np.uint8)
    packed[0, 0] = 0x21      # elements 0, 1 -> codes 1 (0.5), 2 (1.0)
    packed[0, 7] = 0xF7      # elements 14, 15 -> codes 7 (6.0), 15 (-6.0)
    packed[0, 8] = 0x9C      # elements 16, 17 -> codes 12 (-2.0), 9 (-0.5)
    packed[1, 15] = 0x53     # elements 30, 31 -> codes 3 (1.5), 5 (3.0)
    scales = np.array([[0x38, 0x40],       # 1.0, 2.0
                       [0x01, 0x7E]],      # 2^-9 (smallest subnormal), 448
                      np.uint8)
    d = numerics.nvfp4_dequant(packed, scales, 0.25)
    want = np.zeros((2, 32))
    want[0, 0], want[0, 1], want[0, 14], want[0, 15] = 0.5 * 0.25, 1.0 * 0.25, 6.0 * 0.25, -6.0 * 0.25
    want[0, 16], want[0, 17] = -2.0 * 2.0 * 0.25, -0.5 * 2.0 * 0.25
    want[1, 30], want[1, 31] = 1.5 * 448 * 0.25, 3.0 * 448 * 0.25
    assert np.array_equal(d, want)


def test_nvfp4_tensor_scale_is_fp32():
    # the per-tensor scale is an fp32 value: a float64 argument is taken after rounding to fp32
    packed = np.full((1, 8), 0x22, np.uint8)               # every element 1.0
    d = numerics.nvfp4_dequant(packed, np.array([[0x38]], np.uint8), 0.1)
    assert np.all(d == float(np.float32(0.1)))


def test_nvfp4_products_are_exact_in_bf16():
    """Every E2M1 x E4M3 product (finite scale codes) has at most 6 significant bits and lies in
    [2^-10, 2688], so it is a bf16 value: the unscaled weight needs no rounding."""
    for sc in range(256):
        s = numerics.e4m3_value(sc)
        if not np.isfinite(s):
            continue
        for c in range(16):
            p = numerics.e2m1_value(c) * s
            b = synth.f32_to_bf16_bits(np.array([p], np.float32))
            assert numerics.bf16_bits_to_f64(b)[0] == p


def test_nvfp4_synthetic_weights_round_trip_bound():
    """The input generator's NVFP4 encoding: codes decode to within half a grid step (at most one
    E2M1 unit) of each scaled element, or 1/16 of the block maximum where the scale rounded down
    and the element saturated at 6."""
    x = synth.normal_f32((48, 160), 7, 0.02)
    q, s, t = synth.nvfp4_quantize(x)
    assert q.shape == (48, 80) and s.shape == (48, 10) and np.float32(t) == t
    d = numerics.nvfp4_dequant(q, s, t)
    sv = numerics.e4m3_to_f64(s) * t
    bmax = np.abs(x.astype(np.float64)).reshape(48, 10, 16).max(-1)
    bound = np.maximum(sv, bmax / 16.0) * (1 + 1e-6)
    err = np.abs(d - x).reshape(48, 10, 16).max(-1)
    assert np.all(err <= bound)
    assert np.abs(d).max() <= 6 * 448 * t * (1 + 1e-6)


@pytest.mark.parametrize("T,n_in,n_out", [(3, 16, 5), (7, 48, 2), (2, 32, 17)])
def test_nvfp4_weight_products_brute_force(T, n_in, n_out):
    """Forward and dgrad over an NVFP4 weight equal triple loops over weights decoded one element
    at a time with the scalar E2M1 and E4M3 rules."""
    rng = np.random.default_rng(T * 7 + n_in + n_out)
    packed = rng.integers(0, 256, (n_out, n_in // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x50, (n_out, n_in // 16), dtype=np.uint8)
    t = 0.0625
    W = np.empty((n_out, n_in))
    for o in range(n_out):
        for i in range(n_in):
            byte = int(packed[o, i // 2])
            code = (byte >> 4) if i % 2 else (byte & 0xF)
            W[o, i] = numerics.e2m1_value(code) * numerics.e4m3_value(int(scales[o, i // 16])) * t
    X = synth.f32_to_bf16_bits(rng.standard_normal((T, n_in)).astype(np.float32))
    dY = synth.f32_to_bf16_bits(rng.standard_normal((T, n_out)).astype(np.float32))
    np.testing.assert_allclose(linear.linear_fwd_nvfp4w(X, packed, scales, t),
                               linear.fwd_brute(numerics.bf16_bits_to_f64(X), W), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(linear.linear_dgrad_nvfp4w(dY, packed, scales, t),
                               linear.dgrad_brute(numerics.bf16_bits_to_f64(dY), W), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# The parity metric: max|got - ref| / max|ref| over one tensor
# ---------------------------------------------------------------------------------------------

def _rel_err_cases():
    """(got, ref, value) triples worked by hand."""
    return [
        # the largest |ref| is negative and the largest |got - ref| has a negative sign:
        # |diff| = [0, 2, 1] -> 2; max|ref| = 4 -> 0.5
        (np.array([1.0, -6.0, 3.0]), np.array([1.0, -4.0, 2.0]), 0.5),
        # two-dimensional: the maxima are taken over every entry, not per row
        (np.array([[0.0, 1.0], [3.0, 3.5]]), np.array([[0.0, 2.0], [-8.0, 3.0]]), 11.0 / 8.0),
        # identical tensors
        (np.array([[-1.5, 2.0]]), np.array([[-1.5, 2.0]]), 0.0),
        # both all-zero: no error
        (np.zeros((3, 2)), np.zeros((3, 2)), 0.0),
        # empty tensors
        (np.zeros((0, 4)), np.zeros((0, 4)), 0.0),
    ]


def test_rel_err_hand_computed_values():
    for got, ref, want in _rel_err_cases():
        assert linear.rel_err(got, ref) == want, (got, ref)
    # a nonzero result against an all-zero reference can pass no bar
    assert linear.rel_err(np.array([0.0, 1e-30]), np.zeros(2)) == math.inf
    # a power-of-two rescaling of both sides, or a joint sign flip, leaves the metric unchanged
    got, ref, want = _rel_err_cases()[0]
    assert linear.rel_err(-4.0 * got, -4.0 * ref) == want


def test_rel_err_non_finite_results_fail_every_bar():
    ref = np.array([1.0, -2.0, 0.5])
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1] = bad
        e = linear.rel_err(got, ref)
        assert not (e <= 4e-3) and not (e <= 1e-4), (bad, e)


def test_rel_err_pins_catch_planted_slips():
    """Plausible mistakes in the metric each fail one of the hand-worked cases above."""
    def dropped_abs(got, ref):
        return float(np.max(got - ref) / np.max(np.abs(ref)))

    def mean_denominator(got, ref):
        return float(np.max(np.abs(got - ref)) / np.mean(np.abs(ref)))

    def signed_denominator(got, ref):
        return float(np.max(np.abs(got - ref)) / np.max(ref))

    def zero_ref_passes(got, ref):
        den = np.max(np.abs(ref))
        return 0.0 if den == 0 else float(np.max(np.abs(got - ref)) / den)

    for slip in (dropped_abs, mean_denominator, signed_denominator):
        assert any(slip(g, r) != v for g, r, v in _rel_err_cases()[:2]), slip.__name__
    assert zero_ref_passes(np.array([0.0, 1e-30]), np.zeros(2)) != math.inf


# ---------------------------------------------------------------------------------------------
# MXFP8-operand products ([GTP] section 1.3: E4M3 elements, one E8M0 scale per 32 elements)
# ---------------------------------------------------------------------------------------------

def _mx_scalar(codes, scales, r, c):
    """One MXFP8 element by the scalar definitions: E4M3(code) * 2^(scale of block c // 32 - 127)."""
    return numerics.e4m3_value(int(codes[r, c])) * 2.0 ** (int(scales[r, c // 32]) - 127)


def _mx_operands(T, n_in, n_out, seed):
    """Random finite codes; X and W scales from disjoint ranges that also differ block to block,
    so a swapped, transposed or mis-indexed scale array changes the products."""
    rng = np.random.default_rng(seed)
    Xq = rng.integers(0, 256, (T, n_in), dtype=np.uint8)
    Wq = rng.integers(0, 256, (n_out, n_in), dtype=np.uint8)
    for q in (Xq, Wq):
        q[(q & 0x7F) == 0x7F] = 0x3A                           # no NaN codes
    Xs = rng.integers(118, 124, (T, n_in // 32), dtype=np.uint8)
    Ws = rng.integers(128, 134, (n_out, n_in // 32), dtype=np.uint8)
    dY = synth.f32_to_bf16_bits(rng.standard_normal((T, n_out)).astype(np.float32))
    G0 = rng.standard_normal((n_out, n_in))
    return Xq, Xs, Wq, Ws, dY, G0


def _mx_brute(Xq, Xs, Wq, Ws, dY, G0):
    """fwd, dgrad and wgrad-accumulate as triple loops over elements decoded one at a time."""
    T, n_in = Xq.shape
    n_out = Wq.shape[0]
    X = np.array([[_mx_scalar(Xq, Xs, t, i) for i in range(n_in)] for t in range(T)])
    W = np.array([[_mx_scalar(Wq, Ws, o, i) for i in range(n_in)] for o in range(n_out)])
    d = numerics.bf16_bits_to_f64(dY)
    Y = np.array([[sum(X[t, i] * W[o, i] for i in range(n_in)) for o in range(n_out)] for t in range(T)])
    dX = np.array([[sum(d[t, o] * W[o, i] for o in range(n_out)) for i in range(n_in)] for t in range(T)])
    G = np.array([[G0[o, i] + sum(d[t, o] * X[t, i] for t in range(T)) for i in range(n_in)]
                  for o in range(n_out)])
    return Y, dX, G


def _mx_matches(fwd, dgrad, wgrad, case):
    Xq, Xs, Wq, Ws, dY, G0 = case
    Y, dX, G = _mx_brute(*case)
    close = lambda a, b: np.allclose(a, b, rtol=1e-12, atol=1e-12)   # noqa: E731
    return (close(fwd(Xq, Xs, Wq, Ws), Y), close(dgrad(dY, Wq, Ws), dX),
            close(wgrad(G0, Xq, Xs, dY), G))


@pytest.mark.parametrize("T,n_in,n_out", [(3, 64, 5), (2, 96, 3), (5, 32, 7)])
def test_mxfp8_operand_products_brute_force(T, n_in, n_out):
    """linear_fwd_mxfp8, linear_dgrad_mxfp8w and linear_wgrad_accum_mxfp8x equal triple loops over
    operands decoded element by element with the scalar E4M3 and E8M0 rules."""
    case = _mx_operands(T, n_in, n_out, seed=T * 31 + n_in + n_out)
    assert all(_mx_matches(linear.linear_fwd_mxfp8, linear.linear_dgrad_mxfp8w,
                           linear.linear_wgrad_accum_mxfp8x, case))


def test_mxfp8_operand_pins_catch_planted_slips():
    """Plausible mistakes in the three compositions each fail the brute-force comparison."""
    deq, e4m3, e8m0 = numerics.mxfp8_dequant, numerics.e4m3_to_f64, numerics.e8m0_to_f64
    fwd, dgrad, wgrad = linear.linear_fwd_mxfp8, linear.linear_dgrad_mxfp8w, linear.linear_wgrad_accum_mxfp8x
    square = _mx_operands(32, 64, 32, seed=5)      # T == out: the X and W scale arrays can be swapped
    cube = _mx_operands(3, 64, 64, seed=6)         # in == out: W and W^T have the same shape
    slips = {
        "fwd: X and W scales swapped": (square, lambda Xq, Xs, Wq, Ws: linear.linear_fwd(deq(Xq, Ws), deq(Wq, Xs)),
                                        dgrad, wgrad),
        "fwd: W scales ignored": (square, lambda Xq, Xs, Wq, Ws: linear.linear_fwd(deq(Xq, Xs), e4m3(Wq)), dgrad, wgrad),
        "fwd: first block's scale for the whole row": (
            square, lambda Xq, Xs, Wq, Ws: linear.linear_fwd(e4m3(Xq) * e8m0(Xs[:, :1]), deq(Wq, Ws)), dgrad, wgrad),
        "dgrad: W transposed": (cube, fwd, lambda dY, Wq, Ws: linear.linear_dgrad(dY, deq(Wq, Ws).T), wgrad),
        "dgrad: scale exponent off by one": (cube, fwd, lambda dY, Wq, Ws: linear.linear_dgrad(dY, deq(Wq, Ws) * 2.0),
                                             wgrad),
        "wgrad: main_grad dropped": (square, fwd, dgrad, lambda G0, Xq, Xs, dY: linear.linear_wgrad(deq(Xq, Xs), dY)),
        "wgrad: X scales ignored": (square, fwd, dgrad,
                                    lambda G0, Xq, Xs, dY: linear.linear_wgrad_accum(G0, e4m3(Xq), dY)),
    }
    for name, (case, f, d, w) in slips.items():
        assert not all(_mx_matches(f, d, w, case)), name
