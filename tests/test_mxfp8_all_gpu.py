"""GPU parity of the all-MXFP8 step (through the C ABI) against the float64 oracle.

The quantiser is integer/byte work and is compared bit for bit with the oracle's quantiser (codes
and scales, rowwise and transposed columnwise); the fp8 dgrad / wgrad products are compared with
the oracle's products over the same codes, max|gpu - ref| / max|ref| <= 4e-3 (bf16 dX) and
<= 1e-4 (fp32 main_grad).  Small cases element by element, the full-size workload on sampled
rows and entries.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import linear as ol
from oracle import numerics
from synth import configs
from tests.gpu_util import dev_bf16, dev_u8, host_f64, say

import sharded_linear_amd as sl

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3
TOL_F32 = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _bf16_case(R, C, seed):
    """bf16 bits with rows of very different magnitude, plus zero blocks, signed zeros, huge,
    tiny (bf16 subnormal) and exactly representable values."""
    rng = np.random.default_rng(seed)
    x = synth.normal_f32((R, C), seed) * np.exp2(rng.integers(-30, 30, (R, 1))).astype(np.float32)
    x[0, :32] = 0.0                                          # an all-zero row block
    x[:32, min(C - 1, 40)] = -0.0 if R >= 32 else x[:32, min(C - 1, 40)]
    if R > 2:
        x[1, :] = np.float32(3.0e38) * np.sign(x[1, :] + 0.5)                # near the bf16 maximum
        x[2, :] = np.float32(2.0 ** -130) * (1 + np.arange(C) % 5)           # bf16 subnormals
    bits = synth.f32_to_bf16_bits(x)
    return bits


@pytest.mark.parametrize("R,C", [(32, 32), (64, 96), (160, 288), (256, 1024), (4096, 384)])
def test_quantise_bit_exact(R, C):
    say(f"case quantise R={R} C={C}")
    bits = _bf16_case(R, C, R + C)
    xf = numerics.bf16_bits_to_f64(bits)
    qr, sr, qc, sc = sl.sl_mxfp8_quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    wqr, wsr = numerics.mx_quantize(xf)
    wqc, wsc = numerics.mx_quantize_cols(xf)
    assert np.array_equal(qr.cpu().numpy(), wqr) and np.array_equal(sr.cpu().numpy(), wsr)
    assert np.array_equal(qc.cpu().numpy(), wqc) and np.array_equal(sc.cpu().numpy(), wsc)


def test_quantise_beyond_65535_row_tiles():
    """2^23 + 32 rows (65537 row tiles of 128): both copies, checked against the oracle on the
    first rows and on the row blocks around 2^23.  The matrix repeats a [4096, 32] block."""
    R, C = (1 << 23) + 32, 32
    say(f"case quantise R={R} C={C}")
    bits = np.tile(_bf16_case(4096, C, 5), ((R + 4095) // 4096, 1))[:R]
    qr, sr, qc, sc = sl.sl_mxfp8_quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    for lo, hi in ((0, 128), ((1 << 23) - 96, R)):
        xf = numerics.bf16_bits_to_f64(bits[lo:hi])
        wqr, wsr = numerics.mx_quantize(xf)
        wqc, wsc = numerics.mx_quantize_cols(xf)
        assert np.array_equal(qr[lo:hi].cpu().numpy(), wqr) and np.array_equal(sr[lo:hi].cpu().numpy(), wsr)
        assert np.array_equal(qc[:, lo:hi].cpu().numpy(), wqc)
        assert np.array_equal(sc[:, lo // 32:hi // 32].cpu().numpy(), wsc)


@pytest.mark.parametrize("shuffle", [False, True])
def test_quantise_every_bf16_pattern(shuffle):
    """Every finite bf16 bit pattern, laid out as a [2048, 32] matrix (in order, or shuffled so
    that blocks mix magnitudes): rowwise and columnwise codes and scales bit for bit."""
    say(f"case quantise every bf16 pattern shuffle={shuffle}")
    pats = np.array([b for b in range(65536) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)   # 65280
    bits = np.zeros(2048 * 32, np.uint16)
    bits[: pats.size] = np.random.default_rng(3).permutation(pats) if shuffle else pats
    bits = bits.reshape(2048, 32)
    xf = numerics.bf16_bits_to_f64(bits)
    qr, sr, qc, sc = sl.sl_mxfp8_quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    wqr, wsr = numerics.mx_quantize(xf)
    wqc, wsc = numerics.mx_quantize_cols(xf)
    assert np.array_equal(sr.cpu().numpy(), wsr) and np.array_equal(sc.cpu().numpy(), wsc)
    got_r, got_c = qr.cpu().numpy(), qc.cpu().numpy()
    bad = np.argwhere(got_r != wqr)[:5]
    assert bad.size == 0, [(int(bits[r, c]), int(got_r[r, c]), int(wqr[r, c])) for r, c in bad]
    assert np.array_equal(got_c, wqc)


@pytest.mark.parametrize("R,C", [(64, 8), (160, 264)])
def test_quantise_columnwise_only_ragged_cols(R, C):
    """Columnwise copies need only rows % 32 (and cols % 8)."""
    say(f"case quantise cols only R={R} C={C}")
    bits = _bf16_case(R, C, 9 + C)
    qr, sr, qc, sc = sl.sl_mxfp8_quantize(dev_bf16(bits), rows=False)
    torch.cuda.synchronize()
    assert qr is None and sr is None
    wqc, wsc = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(bits))
    assert np.array_equal(qc.cpu().numpy(), wqc) and np.array_equal(sc.cpu().numpy(), wsc)


@pytest.mark.parametrize("R,C", [(100, 64), (33, 320)])
def test_quantise_rowwise_only_ragged_rows(R, C):
    """Rowwise copies need only cols % 32; the columnwise copy is skipped."""
    say(f"case quantise rows only R={R} C={C}")
    bits = _bf16_case(R, C, 7 + R)
    qr, sr, qc, sc = sl.sl_mxfp8_quantize(dev_bf16(bits), cols=False)
    torch.cuda.synchronize()
    assert qc is None and sc is None
    wqr, wsr = numerics.mx_quantize(numerics.bf16_bits_to_f64(bits))
    assert np.array_equal(qr.cpu().numpy(), wqr) and np.array_equal(sr.cpu().numpy(), wsr)


def _quantised_case(T, n_in, n_out, seed):
    X = synth.normal_bf16((T, n_in), seed * 10 + 1)
    W = synth.normal_bf16((n_out, n_in), seed * 10 + 0, synth.W_STD)
    dY = synth.normal_bf16((T, n_out), seed * 10 + 2)
    return X, W, dY


@pytest.mark.parametrize("T,n_in,n_out", [(1, 8, 128), (300, 264, 512), (1000, 520, 256), (513, 2056, 384)])
def test_fp8_dgrad_elementwise(T, n_in, n_out):
    say(f"case fp8 dgrad T={T} in={n_in} out={n_out}")
    _, W, dY = _quantised_case(T, n_in, n_out, T + n_in)
    dYq, dYs, _, _ = sl.sl_mxfp8_quantize(dev_bf16(dY), cols=False)
    _, _, WqT, WsT = sl.sl_mxfp8_quantize(dev_bf16(W), rows=False)
    dX = sl.sl_linear_dgrad_mxfp8(dYq, dYs, WqT, WsT)
    torch.cuda.synchronize()
    q, s = numerics.mx_quantize(numerics.bf16_bits_to_f64(dY))
    qt, st = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(W))
    e = ol.rel_err(host_f64(dX), ol.linear_dgrad_mxfp8(q, s, qt, st))
    say(f"  rel err dX {e:.2e}")
    assert e <= TOL_BF16


@pytest.mark.parametrize("T,n_in,n_out", [(128, 8, 8), (256, 264, 520), (1024, 776, 264), (4096, 264, 520),
                                          (2048, 1032, 2056)])
def test_fp8_wgrad_accum_elementwise(T, n_in, n_out):
    """Unsplit and split-K weight gradients, accumulated onto a nonzero main_grad, twice (the
    workspace then holds the first call's planes)."""
    say(f"case fp8 wgrad T={T} in={n_in} out={n_out} ws={sl.sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out)}")
    X, _, dY = _quantised_case(T, n_in, n_out, T + n_out)
    G0 = synth.normal_f32((n_out, n_in), 5)
    _, _, dYqT, dYsT = sl.sl_mxfp8_quantize(dev_bf16(dY), rows=False)
    _, _, XqT, XsT = sl.sl_mxfp8_quantize(dev_bf16(X), rows=False)
    G = torch.from_numpy(G0).cuda()
    for _ in range(2):
        sl.sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, G)
    torch.cuda.synchronize()
    qd, sd = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(dY))
    qx, sx = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(X))
    want = ol.linear_wgrad_accum_mxfp8(ol.linear_wgrad_accum_mxfp8(G0, qd, sd, qx, sx), qd, sd, qx, sx)
    e = ol.rel_err(host_f64(G), want)
    say(f"  rel err main_grad {e:.2e}")
    assert e <= TOL_F32


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_every_fp8_tile_config(tune, cfg):
    """Each block-scaled fp8 tile configuration (256x256, 128x128, 256x128), forced through
    sl_set_tuning, on the forward, the dgrad and the split-K weight gradient of one ragged shape."""
    T, n_in, n_out = 2176, 1152, 896                 # ragged against 256; 2 K splits in every configuration
    say(f"case fp8 cfg={cfg} T={T} in={n_in} out={n_out}")
    tune(f8=cfg)
    assert sl.sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out) == 2 * n_out * n_in * 4
    X, W, dY = _quantised_case(T, n_in, n_out, 31 + cfg)
    Xf, Wf, dYf = (numerics.bf16_bits_to_f64(a) for a in (X, W, dY))
    Xq, Xs, XqT, XsT = sl.sl_mxfp8_quantize(dev_bf16(X))
    Wq, Ws, WqT, WsT = sl.sl_mxfp8_quantize(dev_bf16(W))
    dYq, dYs, dYqT, dYsT = sl.sl_mxfp8_quantize(dev_bf16(dY))
    G0 = synth.normal_f32((n_out, n_in), 6)
    G = torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd_mxfp8(Xq, Xs, Wq, Ws)
    dX = sl.sl_linear_dgrad_mxfp8(dYq, dYs, WqT, WsT)
    sl.sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, G)
    torch.cuda.synchronize()
    q, s_ = numerics.mx_quantize(Xf)
    wq, ws = numerics.mx_quantize(Wf)
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_mxfp8(q, s_, wq, ws))
    dq, ds = numerics.mx_quantize(dYf)
    wqt, wst = numerics.mx_quantize_cols(Wf)
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad_mxfp8(dq, ds, wqt, wst))
    qd, sd = numerics.mx_quantize_cols(dYf)
    qx, sx = numerics.mx_quantize_cols(Xf)
    e_g = ol.rel_err(host_f64(G), ol.linear_wgrad_accum_mxfp8(G0, qd, sd, qx, sx))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("T,n_in,n_out", [(2560, 1536, 1024), (2560, 2048, 896)])
def test_fp8_scale_groups(tune, cfg, T, n_in, n_out):
    """Contractions whose length is a multiple of 512 load their block scales four stages at a time
    into a double-buffered cache.  Each configuration, forced: the forward, the dgrad (its K = out is a
    multiple of 512 in the first shape only) and a weight gradient in two K splits of 10 stages, so
    the second split starts in the middle of a four-stage group; element by element."""
    say(f"case fp8 scale groups cfg={cfg} T={T} in={n_in} out={n_out}")
    tune(f8=cfg)
    assert sl.sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out) == 2 * n_out * n_in * 4
    X, W, dY = _quantised_case(T, n_in, n_out, 61 + cfg)
    Xf, Wf, dYf = (numerics.bf16_bits_to_f64(a) for a in (X, W, dY))
    Xq, Xs, XqT, XsT = sl.sl_mxfp8_quantize(dev_bf16(X))
    Wq, Ws, WqT, WsT = sl.sl_mxfp8_quantize(dev_bf16(W))
    dYq, dYs, dYqT, dYsT = sl.sl_mxfp8_quantize(dev_bf16(dY))
    G0 = synth.normal_f32((n_out, n_in), 7)
    G = torch.from_numpy(G0).cuda()
    Y = sl.sl_linear_fwd_mxfp8(Xq, Xs, Wq, Ws)
    dX = sl.sl_linear_dgrad_mxfp8(dYq, dYs, WqT, WsT)
    sl.sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, G)
    torch.cuda.synchronize()
    q, s_ = numerics.mx_quantize(Xf)
    wq, ws = numerics.mx_quantize(Wf)
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_mxfp8(q, s_, wq, ws))
    dq, ds = numerics.mx_quantize(dYf)
    wqt, wst = numerics.mx_quantize_cols(Wf)
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad_mxfp8(dq, ds, wqt, wst))
    qd, sd = numerics.mx_quantize_cols(dYf)
    qx, sx = numerics.mx_quantize_cols(Xf)
    e_g = ol.rel_err(host_f64(G), ol.linear_wgrad_accum_mxfp8(G0, qd, sd, qx, sx))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} main_grad {e_g:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16 and e_g <= TOL_F32


@pytest.mark.parametrize("T,n_in,n_out", [(2048, 1032, 776), (4096, 4096, 2048), (2048, 4096, 4096)])
def test_fp8_wgrad_is_deterministic(T, n_in, n_out):
    """The same weight gradient accumulated twice from the same main_grad gives the same bits:
    split-K planes are summed in split order, and the unsplit plans (256x128 and 256x256 tiles)
    do one read-modify-write per element."""
    say(f"case fp8 wgrad determinism T={T} in={n_in} out={n_out} ws={sl.sl_mxfp8_wgrad_workspace_bytes(T, n_in, n_out)}")
    X, _, dY = _quantised_case(T, n_in, n_out, 17 + T)
    _, _, dYqT, dYsT = sl.sl_mxfp8_quantize(dev_bf16(dY), rows=False)
    _, _, XqT, XsT = sl.sl_mxfp8_quantize(dev_bf16(X), rows=False)
    G0 = torch.from_numpy(synth.normal_f32((n_out, n_in), 8)).cuda()
    outs = []
    for _ in range(2):
        G = G0.clone()
        sl.sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, G)
        outs.append(G)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


@pytest.mark.timeout(900)
def test_all_mxfp8_workload_sampled():
    """The all-MXFP8 workload at full size in the benchmark's launch configuration, all 8 micro-batches
    accumulated into one zeroed grad buffer:
    quantisation on the GPU, fwd / dgrad / wgrad on the block-scaled fp8 MFMA; Y and dX checked on
    sampled rows, main_grad on sampled entries (the oracle quantises only the rows and columns
    those need, plus the whole weight)."""
    w = configs.WORKLOADS["c6"]
    buf = sl.ParamAndGradBuffer(w.params, "cuda")
    buf.zero_grad_buffer()
    rng = np.random.default_rng(7)
    state = {}
    for name in w.step_params:
        o, i = w.params[name]
        Wb = configs.weight(w, name)
        buf.param(name).copy_(dev_bf16(Wb))
        Wf = numerics.bf16_bits_to_f64(Wb)
        state[name] = dict(gpu=sl.sl_mxfp8_quantize(buf.param(name)), wr=numerics.mx_quantize(Wf),
                           wc=numerics.mx_quantize_cols(Wf), so=rng.integers(0, o, 256), si=rng.integers(0, i, 256),
                           acc=np.zeros((256, 256)))
    for k in range(w.microbatches):
        for name in w.step_params:
            o, i = w.params[name]
            say(f"  c6 mb={k} {name} [{o},{i}]")
            st = state[name]
            Wqr, Wsr, WqT, WsT = st["gpu"]
            xk, dyk = configs.x(w, name, k), configs.dy(w, name, k)
            Xq, Xs, XqT, XsT = sl.sl_mxfp8_quantize(dev_bf16(xk))
            dYq, dYs, dYqT, dYsT = sl.sl_mxfp8_quantize(dev_bf16(dyk))
            Y = sl.sl_linear_fwd_mxfp8(Xq, Xs, Wqr, Wsr)
            dX = sl.sl_linear_dgrad_mxfp8(dYq, dYs, WqT, WsT)
            sl.sl_linear_wgrad_accum_mxfp8(dYqT, dYsT, XqT, XsT, buf.main_grad(name))
            torch.cuda.synchronize()
            rows = np.unique(np.concatenate([[0, w.tokens - 1], np.random.default_rng(k).integers(0, w.tokens, 48)]))
            xq, xs = numerics.mx_quantize(numerics.bf16_bits_to_f64(xk[rows]))
            dq, ds = numerics.mx_quantize(numerics.bf16_bits_to_f64(dyk[rows]))
            rt = torch.from_numpy(rows).cuda()
            e_y = ol.rel_err(host_f64(Y[rt]), ol.linear_fwd_mxfp8(xq, xs, *st["wr"]))
            e_dx = ol.rel_err(host_f64(dX[rt]), ol.linear_dgrad_mxfp8(dq, ds, *st["wc"]))
            say(f"    rel err Y {e_y:.2e} dX {e_dx:.2e}")
            assert e_y <= TOL_BF16 and e_dx <= TOL_BF16
            # main_grad entries (so, si): columns so of dY and si of X, quantised down the columns
            so, si = st["so"], st["si"]
            cd, cds = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(dyk[:, so]))
            cx, cxs = numerics.mx_quantize_cols(numerics.bf16_bits_to_f64(xk[:, si]))
            st["acc"] = ol.linear_wgrad_accum_mxfp8(st["acc"], cd, cds, cx, cxs)
    for name in w.step_params:
        st = state[name]
        got = host_f64(buf.main_grad(name))[st["so"], st["si"]]
        e = ol.rel_err(got, np.diag(st["acc"]))
        say(f"  c6 {name} main_grad sampled rel err {e:.2e}")
        assert e <= TOL_F32
