"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Bars: max|gpu - ref| / max|ref| <= 4e-3 for bf16 outputs (Y, dX) and <= 1e-4 for the fp32
main_grad, per tensor; layouts, padding and untouched neighbours are compared bit-exactly.
Small cases are compared element by element; the full-size workloads on sampled rows and
entries that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import linear as ol
from oracle import layout as olayout
from oracle import numerics
from synth import configs
from tests.gpu_util import dev_bf16, dev_u8, host_bits, host_f64, say

import sharded_linear_amd as sl

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3
TOL_F32 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sl.sl_linear_fwd  # noqa: B018
    yield
    torch.cuda.synchronize()


def rand_case(T, n_in, n_out, seed):
    X = synth.normal_bf16((T, n_in), seed * 10 + 1)
    W = synth.normal_bf16((n_out, n_in), seed * 10 + 0, synth.W_STD)
    dY = synth.normal_bf16((T, n_out), seed * 10 + 2)
    return X, W, dY


# shapes: (T, in, out) -- ragged tails in every dimension, the 128- and 256-tile configurations,
# split-K and unsplit weight gradients, minimum extents
SMALL = [
    (1, 8, 8), (7, 24, 40), (128, 256, 512), (300, 264, 520), (513, 1032, 776),
    (4104, 264, 520), (1000, 2056, 264), (4100, 264, 3336), (3333, 3336, 4104),
    # weight gradient with 144 tiles of 256x256 and 288 of 256x128: the unsplit 256x128 rule, ragged
    (1000, 4000, 2056),
]


@pytest.mark.parametrize("T,n_in,n_out", SMALL)
def test_fwd_dgrad_wgrad_elementwise(T, n_in, n_out):
    say(f"case T={T} in={n_in} out={n_out}")
    X, W, dY = rand_case(T, n_in, n_out, T + n_in + n_out)
    G0 = synth.normal_f32((n_out, n_in), 99)
    Xd, Wd, dYd = dev_bf16(X), dev_bf16(W), dev_bf16(dY)
    Gd = torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd(Xd, Wd)
    dX = sl.sl_linear_dgrad(dYd, Wd)
    sl.sl_linear_wgrad_accum(Xd, dYd, Gd)
    torch.cuda.synchronize()
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd(X, W))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad(dY, W))
    e_g = ol.rel_err(host_f64(Gd), ol.linear_wgrad_accum(G0, X, dY))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e} ws={sl.sl_wgrad_workspace_bytes(T, n_in, n_out)}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


@pytest.mark.parametrize("cfg", range(25))
@pytest.mark.parametrize("T,n_in,n_out", [(300, 264, 520), (1000, 2056, 264), (2111, 1032, 776), (4104, 264, 520)])
def test_every_tile_config(tune, cfg, T, n_in, n_out):
    """Each direct-to-LDS tile configuration, forced through sl_set_tuning, on ragged shapes."""
    say(f"case cfg={cfg} T={T} in={n_in} out={n_out}")
    tune(gemm=cfg)
    X, W, dY = rand_case(T, n_in, n_out, 31 + cfg)
    G0 = synth.normal_f32((n_out, n_in), 98)
    Xd, Wd, dYd = dev_bf16(X), dev_bf16(W), dev_bf16(dY)
    Gd = torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd(Xd, Wd)
    dX = sl.sl_linear_dgrad(dYd, Wd)
    sl.sl_linear_wgrad_accum(Xd, dYd, Gd)
    torch.cuda.synchronize()
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd(X, W))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad(dY, W))
    e_g = ol.rel_err(host_f64(Gd), ol.linear_wgrad_accum(G0, X, dY))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


@pytest.mark.parametrize("T,n_in,n_out", [(300, 264, 520), (1000, 2056, 264), (2111, 1032, 776), (4104, 264, 520),
                                          (520, 4104, 1544), (1024, 2048, 1536)])
def test_forward_256x192_tiles(tune, T, n_in, n_out):
    """The forward-only 256x192 configuration (cfg 25), forced, on ragged shapes: N not a multiple of
    192, the last k stage partial, M edges inside a tile; element by element against the oracle."""
    say(f"case fwd cfg=25 T={T} in={n_in} out={n_out}")
    tune(fwd=25)
    X, W, _ = rand_case(T, n_in, n_out, 51)
    Y = sl.sl_linear_fwd(dev_bf16(X), dev_bf16(W))
    torch.cuda.synchronize()
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd(X, W))
    say(f"  rel err Y {e_y:.2e}")
    assert e_y <= TOL_BF16


# (T, in, out) whose forward, dgrad or weight gradient has 272 or 288 tiles of 256x256: split along N
# or along M, one shape per product and direction
REGION_SHAPES = [(4096, 256, 4352), (4224, 512, 4096), (4096, 4352, 256), (4224, 4096, 512), (256, 4352, 4096),
                 (320, 4096, 4480)]


@pytest.mark.parametrize("T,n_in,n_out", REGION_SHAPES)
def test_whole_rounds_plus_tail_regions(T, n_in, n_out):
    """Shapes whose 256x256 tiles make one whole round plus a partial one run as two launches (whole
    rounds of 256x256 tiles, then the rest on 256x128 tiles) -- split along N or along M, for each
    product: element by element against the oracle, and the weight gradient stays deterministic."""
    say(f"case regions T={T} in={n_in} out={n_out}")
    X, W, dY = rand_case(T, n_in, n_out, 41)
    G0 = synth.normal_f32((n_out, n_in), 42)
    Xd, Wd, dYd = dev_bf16(X), dev_bf16(W), dev_bf16(dY)
    Ga, Gb = torch.from_numpy(G0).cuda(), torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd(Xd, Wd)
    dX = sl.sl_linear_dgrad(dYd, Wd)
    sl.sl_linear_wgrad_accum(Xd, dYd, Ga)
    sl.sl_linear_wgrad_accum(Xd, dYd, Gb)
    torch.cuda.synchronize()
    assert torch.equal(Ga.view(torch.int32), Gb.view(torch.int32))
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd(X, W))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad(dY, W))
    e_g = ol.rel_err(host_f64(Ga), ol.linear_wgrad_accum(G0, X, dY))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


def test_c1_two_microbatches_into_buffer_view():
    w = configs.WORKLOADS["c1"]
    say("case c1")
    buf = sl.ParamAndGradBuffer({"weight": (512, 256)}, "cuda", bucket_size=None)
    assert buf.numel == 131072 and buf.numel % 64 == 0 and buf.index["weight"][:2] == (0, 131072)
    W = configs.weight(w, "weight")
    buf.param("weight").copy_(dev_bf16(W))
    buf.zero_grad_buffer()
    Xs = [configs.x(w, "weight", k) for k in range(2)]
    dYs = [configs.dy(w, "weight", k) for k in range(2)]
    Ys, dXs = [], []
    for X, dY in zip(Xs, dYs):
        Ys.append(sl.sl_linear_fwd(dev_bf16(X), buf.param("weight")))
        dXs.append(sl.sl_linear_dgrad(dev_bf16(dY), buf.param("weight")))
        sl.sl_linear_wgrad_accum(dev_bf16(X), dev_bf16(dY), buf.main_grad("weight"))
    torch.cuda.synchronize()
    rY, rdX, rG = ol.step(W, Xs, dYs)
    for k in range(2):
        assert ol.rel_err(host_f64(Ys[k]), rY[k]) <= TOL_BF16
        assert ol.rel_err(host_f64(dXs[k]), rdX[k]) <= TOL_BF16
    assert ol.rel_err(host_f64(buf.main_grad("weight")), rG) <= TOL_F32
    # same data twice: a deterministic kernel gives exactly twice the single accumulation
    buf.zero_grad_buffer()
    sl.sl_linear_wgrad_accum(dev_bf16(Xs[0]), dev_bf16(dYs[0]), buf.main_grad("weight"))
    torch.cuda.synchronize()
    once = buf.main_grad("weight").clone()
    sl.sl_linear_wgrad_accum(dev_bf16(Xs[0]), dev_bf16(dYs[0]), buf.main_grad("weight"))
    torch.cuda.synchronize()
    assert torch.equal(buf.main_grad("weight"), 2 * once)


def test_exact_special_cases_bitwise():
    say("case exact special cases")
    rng = np.random.default_rng(5)
    T, n_in, n_out = 96, 264, 136
    W = synth.normal_bf16((n_out, n_in), 5, 1.0)
    X = np.zeros((T, n_in), np.float32)
    cols = rng.integers(0, n_in, size=T)
    X[np.arange(T), cols] = 1.0
    Y = host_f64(sl.sl_linear_fwd(dev_bf16(synth.f32_to_bf16_bits(X)), dev_bf16(W)))
    Wf = ol.linear_fwd(np.eye(n_in), W)          # = W^T as float64, exact
    assert np.array_equal(Y, Wf[cols])            # row t of Y is column cols[t] of W
    dY = np.zeros((T, n_out), np.float32)
    rows = rng.integers(0, n_out, size=T)
    dY[np.arange(T), rows] = 1.0
    dX = host_f64(sl.sl_linear_dgrad(dev_bf16(synth.f32_to_bf16_bits(dY)), dev_bf16(W)))
    assert np.array_equal(dX, ol.linear_dgrad(np.eye(n_out), W)[rows])
    # T = 1: the wgrad is an outer product of bf16 values, exact in fp32
    x1 = synth.normal_bf16((1, n_in), 6)
    g1 = synth.normal_bf16((1, n_out), 7)
    G = torch.zeros((n_out, n_in), dtype=torch.float32, device="cuda")
    sl.sl_linear_wgrad_accum(dev_bf16(x1), dev_bf16(g1), G)
    assert np.array_equal(host_f64(G), ol.linear_wgrad(x1, g1))


def test_empty_and_degenerate():
    say("case empty and degenerate")
    W = dev_bf16(synth.normal_bf16((16, 8), 1))
    X0 = torch.empty((0, 8), dtype=torch.bfloat16, device="cuda")
    dY0 = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    assert sl.sl_linear_fwd(X0, W).shape == (0, 16)
    assert sl.sl_linear_dgrad(dY0, W).shape == (0, 8)
    G = torch.full((16, 8), 3.0, device="cuda")
    sl.sl_linear_wgrad_accum(X0, dY0, G)        # T = 0 leaves main_grad as it was
    torch.cuda.synchronize()
    assert torch.equal(G, torch.full((16, 8), 3.0, device="cuda"))


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_operand_beyond_direct_load_extent(which):
    """One operand of 2 GiB or more: too large for the direct HBM->LDS loads' 32-bit offsets, so
    the GEMM runs on the register-staged kernel.  The big operand repeats a seeded block of P rows
    (plus a ragged tail of R rows), which lets the oracle check fwd / dgrad on sampled rows and
    the weight gradient exactly as reps x (block product) + tail product."""
    P, reps, R = 4096, 64, 520
    T = P * reps + R                       # 262,664 rows
    big, small = 4096, 64                  # 262,664 x 4096 bf16 = 2.15 GB
    say(f"case big operand {which}: T={T} big={big} small={small}")
    blk_big = synth.normal_bf16((P, big), 7001)
    blk_small = synth.normal_bf16((P, small), 7002)

    def tiled(blk):
        d = dev_bf16(blk)
        return torch.cat([d.repeat(reps, 1), d[:R]], dim=0)

    rows = np.r_[0:40, P * 17 + 5:P * 17 + 45, T - 40:T]
    if which == "fwd":                     # X [T, big] huge, W [small, big]
        W = synth.normal_bf16((small, big), 7003, synth.W_STD)
        X = tiled(blk_big)
        Y = sl.sl_linear_fwd(X, dev_bf16(W))
        torch.cuda.synchronize()
        ref = ol.linear_fwd(blk_big[rows % P], W)
        assert ol.rel_err(host_f64(Y[torch.as_tensor(rows, device="cuda")]), ref) <= TOL_BF16
    elif which == "dgrad":                 # dY [T, big] huge, W [big, small]
        W = synth.normal_bf16((big, small), 7004, synth.W_STD)
        dY = tiled(blk_big)
        dX = sl.sl_linear_dgrad(dY, dev_bf16(W))
        torch.cuda.synchronize()
        ref = ol.linear_dgrad(blk_big[rows % P], W)
        assert ol.rel_err(host_f64(dX[torch.as_tensor(rows, device="cuda")]), ref) <= TOL_BF16
    else:                                  # X [T, big] huge, dY [T, small]: main_grad [small, big]
        X, dY = tiled(blk_big), tiled(blk_small)
        G = torch.zeros((small, big), device="cuda")
        sl.sl_linear_wgrad_accum(X, dY, G)
        torch.cuda.synchronize()
        ref = reps * ol.linear_wgrad(blk_big, blk_small) + ol.linear_wgrad(blk_big[:R], blk_small[:R])
        assert ol.rel_err(host_f64(G), ref) <= TOL_F32


def test_mxfp8_fwd_operand_beyond_direct_load_extent():
    """MXFP8 forward with Xq of 2 GiB or more: the block-scaled kernel's direct loads cannot
    address it, so the call runs on the register-staged kernel that dequantises on load.  Xq
    repeats a seeded block of P rows (plus a ragged tail of R rows); Y is checked on sampled rows."""
    P, reps, R = 4096, 64, 520
    T, n_in, n_out = P * reps + R, 8192, 64          # 262,664 x 8192 codes = 2.15 GB
    say(f"case big mxfp8 fwd: T={T} in={n_in} out={n_out}")
    Xb, Sb = synth.mxfp8_normal((P, n_in), 7011)
    Wq, Ws = synth.mxfp8_normal((n_out, n_in), 7012, synth.W_STD)
    xd, sd = dev_u8(Xb), dev_u8(Sb)
    Xq = torch.cat([xd.repeat(reps, 1), xd[:R]], dim=0)
    Xs = torch.cat([sd.repeat(reps, 1), sd[:R]], dim=0)
    Y = sl.sl_linear_fwd_mxfp8(Xq, Xs, dev_u8(Wq), dev_u8(Ws))
    torch.cuda.synchronize()
    rows = np.r_[0:40, P * 17 + 5:P * 17 + 45, T - 40:T]
    ref = ol.linear_fwd_mxfp8(Xb[rows % P], Sb[rows % P], Wq, Ws)
    assert ol.rel_err(host_f64(Y[torch.as_tensor(rows, device="cuda")]), ref) <= TOL_BF16


def test_neighbours_and_padding_untouched():
    """A wgrad into one view of grad_data leaves every other element bit-identical."""
    say("case neighbours and padding")
    shapes = {"a": (136, 264), "b": (520, 264), "c": (8, 8)}
    buf = sl.ParamAndGradBuffer(shapes, "cuda", bucket_size=None)
    ref = olayout.build_layout([136 * 264, 520 * 264, 64], bucket_size=None)
    assert [buf.index[k][:2] for k in shapes] == list(zip(ref.start, ref.end)) and buf.numel == ref.numel
    sentinel = torch.full((buf.numel,), -7.25, device="cuda")
    buf.grad_data.copy_(sentinel)
    X, W, dY = rand_case(4104, 264, 520, 3)       # split-K path
    sl.sl_linear_wgrad_accum(dev_bf16(X), dev_bf16(dY), buf.main_grad("b"))
    torch.cuda.synchronize()
    s, e, _ = buf.index["b"]
    g = buf.grad_data
    assert torch.equal(g[:s], sentinel[:s]) and torch.equal(g[e:], sentinel[e:])
    want = ol.linear_wgrad_accum(np.full((520, 264), -7.25), X, dY)
    assert ol.rel_err(host_f64(buf.main_grad("b")), want) <= TOL_F32


def test_workspace_reused_across_shapes():
    """One workspace serves split-K calls of different shapes in any order; its initial contents
    (here all-ones bytes, a NaN pattern for fp32) never reach the result."""
    say("case workspace reuse")
    cases = [(4104, 264, 520), (1000, 2056, 264), (4100, 288, 3336), (4104, 264, 520)]
    need = max(sl.sl_wgrad_workspace_bytes(*c) for c in cases)
    assert all(sl.sl_wgrad_workspace_bytes(*c) > 0 for c in cases)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for T, n_in, n_out in cases:
        X, W, dY = rand_case(T, n_in, n_out, 77)
        G = torch.zeros((n_out, n_in), device="cuda")
        sl.sl_linear_wgrad_accum(dev_bf16(X), dev_bf16(dY), G, workspace=ws)
        torch.cuda.synchronize()
        e = ol.rel_err(host_f64(G), ol.linear_wgrad(X, dY))
        say(f"  T={T} in={n_in} out={n_out} rel err {e:.2e}")
        assert e <= TOL_F32


def test_wgrad_is_deterministic():
    say("case determinism")
    X, W, dY = rand_case(8192, 1024, 2048, 11)   # split-K path at a C3-like shape
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    outs = []
    for _ in range(3):
        G = torch.zeros((2048, 1024), device="cuda")
        sl.sl_linear_wgrad_accum(Xd, dYd, G)
        outs.append(G)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def _check_non_finite(got, ref, tol):
    """NaN and infinity in the same places (infinities with the same sign); finite entries to tol."""
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf)
    assert np.array_equal(np.sign(got[inf]), np.sign(ref[inf]))
    fin = np.isfinite(ref)
    assert ol.rel_err(got[fin], ref[fin]) <= tol
    return int(np.isnan(ref).sum()), int(inf.sum())


@pytest.mark.parametrize("T,n_in,n_out", [(300, 264, 520), (2048, 1024, 1536)])
def test_nan_and_inf_propagate(T, n_in, n_out):
    """NaN and +-inf in X, in dY and in the old main_grad reach exactly the outputs the definition
    says (a NaN row of X gives a NaN row of Y and a NaN column of main_grad, ...), through the
    unsplit and (second shape) the split-K weight gradient; the finite outputs keep parity."""
    say(f"case non-finite T={T} in={n_in} out={n_out} ws={sl.sl_wgrad_workspace_bytes(T, n_in, n_out)}")
    X, W, dY = rand_case(T, n_in, n_out, 61)
    rng = np.random.default_rng(62)
    t = rng.choice(T, 4, replace=False)
    i = rng.choice(n_in, 4, replace=False)
    o = rng.choice(n_out, 4, replace=False)
    X[t[0], i[0]] = 0x7FC0                 # NaN
    X[t[1], i[1]] = 0x7F80                 # +inf
    dY[t[2], o[0]] = 0x7FC0                # NaN
    dY[t[3], o[1]] = 0xFF80                # -inf
    G0 = synth.normal_f32((n_out, n_in), 63)
    G0[o[2], i[2]] = np.nan
    G0[o[3], i[3]] = -np.inf
    Xd, Wd, dYd = dev_bf16(X), dev_bf16(W), dev_bf16(dY)
    Gd = torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd(Xd, Wd)
    dX = sl.sl_linear_dgrad(dYd, Wd)
    sl.sl_linear_wgrad_accum(Xd, dYd, Gd)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        ry, rdx, rg = ol.linear_fwd(X, W), ol.linear_dgrad(dY, W), ol.linear_wgrad_accum(G0, X, dY)
    ny = _check_non_finite(host_f64(Y), ry, TOL_BF16)
    ndx = _check_non_finite(host_f64(dX), rdx, TOL_BF16)
    ng = _check_non_finite(host_f64(Gd), rg, TOL_F32)
    say(f"  (NaN, inf) counts: Y {ny} dX {ndx} main_grad {ng}")
    assert ny[0] == n_out and ny[1] > 0 and ndx[0] == n_in and ng[0] >= n_in + n_out - 1


def test_grad_buffer_zero_fill():
    say("case zero fill")
    for n in (1, 3, 4, 1023, 1 << 20, (1 << 20) + 5):
        g = torch.full((n,), 5.0, device="cuda")
        sl.sl_grad_buffer_zero(g)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(g)) == 0


def test_autograd_glue():
    """forward saves (input, weight); backward returns dX and no weight grad, fills main_grad."""
    say("case autograd")
    buf = sl.ParamAndGradBuffer({"fc1": (264, 136), "fc2": (136, 264)}, "cuda", bucket_size=None)
    W1 = synth.normal_bf16((264, 136), 1, synth.W_STD)
    W2 = synth.normal_bf16((136, 264), 2, synth.W_STD)
    p1 = buf.attach("fc1", torch.nn.Parameter(dev_bf16(W1).clone()))
    p2 = buf.attach("fc2", torch.nn.Parameter(dev_bf16(W2).clone()))
    assert p1.data_ptr() == buf.param("fc1").data_ptr()
    X = synth.normal_bf16((4, 50, 136), 3)        # [s, b, h]
    dY = synth.normal_bf16((4, 50, 136), 4)
    x = dev_bf16(X).requires_grad_(True)
    z = sl.linear_with_grad_accumulation(x, p1)
    z.retain_grad()
    y = sl.linear_with_grad_accumulation(z, p2)
    y.backward(dev_bf16(dY))
    torch.cuda.synchronize()
    assert p1.grad is None and p2.grad is None
    assert p1.grad_added_to_main_grad and p2.grad_added_to_main_grad
    Xm, dYm = X.reshape(200, 136), dY.reshape(200, 136)
    Zb = host_bits(z).reshape(200, 264)           # what fc2 consumed (bf16)
    dZb = host_bits(z.grad).reshape(200, 264)     # what fc1's backward consumed (bf16)
    assert ol.rel_err(host_f64(z).reshape(200, 264), ol.linear_fwd(Xm, W1)) <= TOL_BF16
    assert ol.rel_err(host_f64(y).reshape(200, 136), ol.linear_fwd(Zb, W2)) <= TOL_BF16
    assert ol.rel_err(host_f64(z.grad).reshape(200, 264), ol.linear_dgrad(dYm, W2)) <= TOL_BF16
    assert ol.rel_err(host_f64(x.grad).reshape(200, 136), ol.linear_dgrad(dZb, W1)) <= TOL_BF16
    assert ol.rel_err(host_f64(buf.main_grad("fc2")), ol.linear_wgrad(Zb, dYm)) <= TOL_F32
    assert ol.rel_err(host_f64(buf.main_grad("fc1")), ol.linear_wgrad(Xm, dZb)) <= TOL_F32


# ---------------------------------------------------------------------------------------------
# MXFP8 operand variants
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("T,n_in,n_out", [(1, 32, 8), (300, 288, 520), (4104, 256, 520), (4100, 288, 3336),
                                          (1000, 384, 776), (4100, 512, 3336)])
def test_mxfp8_elementwise(T, n_in, n_out):
    say(f"case mxfp8 T={T} in={n_in} out={n_out}")
    Xq, Xs = synth.mxfp8_normal((T, n_in), 21)
    Wq, Ws = synth.mxfp8_normal((n_out, n_in), 22, synth.W_STD)
    dY = synth.normal_bf16((T, n_out), 23)
    G0 = synth.normal_f32((n_out, n_in), 24)
    Y = sl.sl_linear_fwd_mxfp8(dev_u8(Xq), dev_u8(Xs), dev_u8(Wq), dev_u8(Ws))
    dX = sl.sl_linear_dgrad_mxfp8w(dev_bf16(dY), dev_u8(Wq), dev_u8(Ws))
    G = torch.from_numpy(G0).cuda()
    sl.sl_linear_wgrad_accum_mxfp8x(dev_u8(Xq), dev_u8(Xs), dev_bf16(dY), G)
    torch.cuda.synchronize()
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_mxfp8(Xq, Xs, Wq, Ws))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad_mxfp8w(dY, Wq, Ws))
    e_g = ol.rel_err(host_f64(G), ol.linear_wgrad_accum_mxfp8x(G0, Xq, Xs, dY))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


@pytest.mark.parametrize("cfg", range(3))
@pytest.mark.parametrize("T,n_in,n_out", [(300, 384, 520), (1000, 512, 776), (2050, 1024, 264), (4100, 256, 3336)])
def test_mxfp8_fwd_every_config(tune, cfg, T, n_in, n_out):
    """Each block-scaled fp8 forward configuration, forced through sl_set_tuning, on ragged M/N."""
    say(f"case mxfp8 fwd cfg={cfg} T={T} in={n_in} out={n_out}")
    tune(f8=cfg)
    Xq, Xs = synth.mxfp8_normal((T, n_in), 31 + cfg)
    Wq, Ws = synth.mxfp8_normal((n_out, n_in), 32 + cfg, synth.W_STD)
    Y = sl.sl_linear_fwd_mxfp8(dev_u8(Xq), dev_u8(Xs), dev_u8(Wq), dev_u8(Ws))
    torch.cuda.synchronize()
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_mxfp8(Xq, Xs, Wq, Ws))
    say(f"  rel err Y {e_y:.2e}")
    assert e_y <= TOL_BF16


@pytest.mark.parametrize("n_in", [32, 128])
def test_mxfp8_all_codes_decode_exactly(n_in):
    """Every finite E4M3 code under several scales: a one-hot fwd returns the decoded value
    (in = 32: register-dequantising kernel; in = 128: block-scaled fp8 MFMA)."""
    say(f"case mxfp8 decode table in={n_in}")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254 codes
    n_out = 256
    Wq = np.zeros((n_out, n_in), np.uint8)
    Wq[: codes.size, n_in - 1] = codes                                               # last block
    for s in (100, 120, 127, 135):
        Ws = np.full((n_out, n_in // 32), 127, np.uint8)
        Ws[:, -1] = s
        Xq = np.zeros((1, n_in), np.uint8); Xq[0, n_in - 1] = 0x38                   # 1.0
        Xs = np.full((1, n_in // 32), 127, np.uint8)
        Y = host_f64(sl.sl_linear_fwd_mxfp8(dev_u8(Xq), dev_u8(Xs), dev_u8(Wq), dev_u8(Ws)))[0]
        want = ol.linear_fwd_mxfp8(Xq, Xs, Wq, Ws)[0]
        assert np.array_equal(Y, want), s


@pytest.mark.parametrize("rows,cols", [(7, 32), (254, 256), (300, 1024)])
def test_mxfp8_dequantize_bit_exact(rows, cols):
    """sl_mxfp8_dequantize against the oracle's decode, bit for bit: every finite E4M3 code under
    block scales from 2^-27 to 2^8 (all results normal bf16), ragged row counts."""
    say(f"case mxfp8 dequantize rows={rows} cols={cols}")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rng = np.random.default_rng(rows + cols)
    q = codes[rng.integers(0, codes.size, (rows, cols))]
    q.reshape(-1)[: min(codes.size, q.size)] = codes[: min(codes.size, q.size)]
    s = rng.integers(100, 136, (rows, cols // 32)).astype(np.uint8)
    out = sl.sl_mxfp8_dequantize(dev_u8(q), dev_u8(s))
    torch.cuda.synchronize()
    want = synth.f32_to_bf16_bits(numerics.mxfp8_dequant(q, s).astype(np.float32))
    assert np.array_equal(host_bits(out), want)


def test_mxfp8_weight_expanded_once_matches_per_call_dgrad():
    """A step that expands the MXFP8 weight once and runs the bf16 dgrad on it gives the per-call
    entry point's dX bit for bit (the same exact expansion feeds the same GEMM)."""
    T, n_in, n_out = 1000, 1024, 776
    say(f"case mxfp8 weight expanded once T={T} in={n_in} out={n_out}")
    Wq, Ws = synth.mxfp8_normal((n_out, n_in), 61, synth.W_STD)
    dY = synth.normal_bf16((T, n_out), 62)
    Wqd, Wsd, dYd = dev_u8(Wq), dev_u8(Ws), dev_bf16(dY)
    Wd = sl.sl_mxfp8_dequantize(Wqd, Wsd)
    a = sl.sl_linear_dgrad(dYd, Wd)
    b = sl.sl_linear_dgrad_mxfp8w(dYd, Wqd, Wsd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    e = ol.rel_err(host_f64(a), ol.linear_dgrad_mxfp8w(dY, Wq, Ws))
    say(f"  rel err dX {e:.2e}")
    assert e <= TOL_BF16


def test_mxfp8_dequantised_operand_exact():
    """The dequantised MXFP8 operand of dgrad and wgrad, bit for bit: with dY = I (T = out), dgrad
    returns deq(Wq) and the weight gradient returns deq(Xq), each element one exact product.
    Every finite E4M3 code appears under each of four block scales."""
    say("case mxfp8 dequantised operand, all codes")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254 codes
    n = 256                                   # out = T = 256 rows, in = 4 blocks of 64 codes
    q = np.zeros((n, 256), np.uint8)
    q.reshape(-1)[: codes.size * 4] = np.tile(codes, 4)
    sc = np.empty((n, 8), np.uint8)
    sc[:] = np.array([100, 120, 127, 135, 127, 135, 100, 120], np.uint8)
    eye = np.zeros((n, n), np.float32)
    np.fill_diagonal(eye, 1.0)
    I = dev_bf16(synth.f32_to_bf16_bits(eye))
    ws = torch.zeros(sl.sl_mxfp8_workspace_bytes(n, 256, n), dtype=torch.uint8, device="cuda")
    # dgrad: dX[T=n, in] = I . deq(Wq[out=n, in])
    dX = sl.sl_linear_dgrad_mxfp8w(I, dev_u8(q), dev_u8(sc), workspace=ws)
    # weight gradient: main_grad[out=n, in] += I^T . deq(Xq[T=n, in])
    G = torch.zeros((n, 256), device="cuda")
    sl.sl_linear_wgrad_accum_mxfp8x(dev_u8(q), dev_u8(sc), I, G, workspace=ws)
    torch.cuda.synchronize()
    from oracle import numerics
    want = numerics.mxfp8_dequant(q, sc)
    assert np.array_equal(host_f64(dX), want)
    assert np.array_equal(host_f64(G), want)


# ---------------------------------------------------------------------------------------------
# Full-size workloads (launch configuration of the benchmark), sampled against the oracle
# ---------------------------------------------------------------------------------------------

def _sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=k)]))


def run_workload_sampled(key, mbs=None):
    w = configs.WORKLOADS[key]
    mbs = w.microbatches if mbs is None else mbs
    buf = sl.ParamAndGradBuffer(w.params, "cuda")
    ref = olayout.build_layout([o * i for o, i in w.params.values()], bucket_size=olayout.default_bucket_size(1))
    for j, name in enumerate(w.params):
        assert buf.index[name] == (ref.start[j], ref.end[j], ref.bucket_id[j])
    assert buf.numel == ref.numel
    buf.zero_grad_buffer()
    weights = {}
    for name in w.step_params:
        wt = configs.weight(w, name)
        weights[name] = wt
        if not w.mxfp8:
            buf.param(name).copy_(dev_bf16(wt))
    # sampled main_grad entries (so[j], si[j]): the oracle accumulates the [256, 256] block of
    # main_grad over rows so and columns si, whose diagonal holds them
    samples = {}
    for name in w.step_params:
        o, i = w.params[name]
        rng = np.random.default_rng(7)
        samples[name] = (rng.integers(0, o, 256), rng.integers(0, i, 256), np.zeros((256, 256)))
    errs = []
    for k in range(mbs):
        for name in w.step_params:
            o, i = w.params[name]
            say(f"  {key} mb={k} {name} [{o},{i}]")
            xk, dyk = configs.x(w, name, k), configs.dy(w, name, k)
            rows = _sample_rows(w.tokens, 48, k)
            if w.mxfp8:
                (Xq, Xs), (Wq, Ws) = xk, weights[name]
                Wqd, Wsd = dev_u8(Wq), dev_u8(Ws)
                Y = sl.sl_linear_fwd_mxfp8(dev_u8(Xq), dev_u8(Xs), Wqd, Wsd)
                dX = sl.sl_linear_dgrad_mxfp8w(dev_bf16(dyk), Wqd, Wsd)
                sl.sl_linear_wgrad_accum_mxfp8x(dev_u8(Xq), dev_u8(Xs), dev_bf16(dyk), buf.main_grad(name))
                Yr = ol.linear_fwd_mxfp8(Xq[rows], Xs[rows], Wq, Ws)
                dXr = ol.linear_dgrad_mxfp8w(dyk[rows], Wq, Ws)
                xf = ol.mxfp8_dequant(Xq, Xs)          # the exact X the wgrad contracts with
            else:
                Wd = buf.param(name)
                Xd = dev_bf16(xk)
                dYd = dev_bf16(dyk)
                Y = sl.sl_linear_fwd(Xd, Wd)
                dX = sl.sl_linear_dgrad(dYd, Wd)
                sl.sl_linear_wgrad_accum(Xd, dYd, buf.main_grad(name))
                Yr = ol.linear_fwd(xk[rows], weights[name])
                dXr = ol.linear_dgrad(dyk[rows], weights[name])
                xf = xk
            torch.cuda.synchronize()
            errs.append(ol.rel_err(host_f64(Y[torch.from_numpy(rows).cuda()]), Yr))
            errs.append(ol.rel_err(host_f64(dX[torch.from_numpy(rows).cuda()]), dXr))
            so, si, acc = samples[name]
            samples[name] = (so, si, ol.linear_wgrad_accum(acc, xf[:, si], dyk[:, so]))
            assert errs[-1] <= TOL_BF16 and errs[-2] <= TOL_BF16, (key, k, name, errs[-2:])
    for name in w.step_params:
        so, si, acc = samples[name]
        got = host_f64(buf.main_grad(name))[so, si]
        e = ol.rel_err(got, np.diag(acc))
        say(f"  {key} {name} main_grad sampled rel err {e:.2e}")
        assert e <= TOL_F32
    # padding and the grad views of params outside the step stay zero
    g = buf.grad_data
    covered = torch.zeros(buf.numel, dtype=torch.bool, device="cuda")
    for name in w.step_params:
        s, e, _ = buf.index[name]
        covered[s:e] = True
    assert int(torch.count_nonzero(g[~covered])) == 0
    say(f"  {key} max bf16 sampled rel err {max(errs):.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_full_size_workload_sampled(key):
    """Every micro-batch of the workload (8 for c2 and c5: main_grad zeroed once, then accumulated
    over all of them with no reduction in between) in the benchmark's launch configuration."""
    say(f"case workload {key}")
    run_workload_sampled(key)
