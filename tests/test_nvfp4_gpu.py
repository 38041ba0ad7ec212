"""GPU parity of the NVFP4-weight path (through the C ABI) against the float64 oracle.

Materialisation is byte work with an exact result (every E2M1 x E4M3 product is a bf16 value), so
it is compared bit for bit with the oracle's decode; the forward and dgrad products over the
materialised weight and the fp32 tensor scale are compared with the oracle's products,
max|gpu - ref| / max|ref| <= 4e-3 per bf16 tensor.  Small cases element by element, the
full-size workload on sampled rows.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import linear as ol
from oracle import numerics
from synth import configs
from tests.gpu_util import dev_bf16, dev_u8, host_bits, host_f64, say

import sharded_linear_amd as sl

pytestmark = pytest.mark.gpu

TOL_BF16 = 4e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    yield
    torch.cuda.synchronize()


def _want_bits(packed, scales):
    """bf16 patterns of the oracle's unscaled decode (exact products, so the conversion is too)."""
    return synth.f32_to_bf16_bits(numerics.nvfp4_dequant(packed, scales, 1.0).astype(np.float32))


def test_materialize_every_code_with_every_scale():
    """Each of the 16 codes under each of the 254 finite scale bytes, in both nibble positions."""
    say("case materialise: every code x every finite scale")
    sc = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    rows = sc.size
    lo = np.arange(16, dtype=np.uint8)
    row = np.concatenate([lo[0::2] | (lo[1::2] << 4), lo[::-1][0::2] | (lo[::-1][1::2] << 4)])   # 32 codes
    packed = np.tile(row, (rows, 1))
    scales = np.stack([sc, sc[::-1]], axis=1)
    Wm = sl.sl_nvfp4_materialize(dev_u8(packed), dev_u8(scales))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Wm), _want_bits(packed, scales))


def test_materialize_nan_scale():
    say("case materialise: NaN scale bytes")
    packed = np.full((2, 8), 0x52, np.uint8)
    scales = np.array([[0x7F], [0xFF]], np.uint8)
    Wm = sl.sl_nvfp4_materialize(dev_u8(packed), dev_u8(scales))
    torch.cuda.synchronize()
    assert torch.isnan(Wm.float()).all()


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (300, 1040), (4097, 272)])
def test_materialize_random_bytes(rows, cols):
    say(f"case materialise rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 3 + cols)
    packed = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, cols // 16), dtype=np.uint8) | (rng.integers(0, 2, (rows, cols // 16),
                                                                                          dtype=np.uint8) << 7)
    Wm = sl.sl_nvfp4_materialize(dev_u8(packed), dev_u8(scales))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Wm), _want_bits(packed, scales))


def _nvfp4_case(T, n_in, n_out, seed):
    q, s, t = synth.nvfp4_normal((n_out, n_in), seed * 10, synth.W_STD)
    X = synth.normal_bf16((T, n_in), seed * 10 + 1)
    dY = synth.normal_bf16((T, n_out), seed * 10 + 2)
    return q, s, t, X, dY


def _run(q, s, t, X, dY):
    Wm = sl.sl_nvfp4_materialize(dev_u8(q), dev_u8(s))
    Y = sl.sl_linear_fwd_nvfp4w(dev_bf16(X), Wm, t)
    dX = sl.sl_linear_dgrad_nvfp4w(dev_bf16(dY), Wm, t)
    torch.cuda.synchronize()
    return Y, dX


@pytest.mark.parametrize("T,n_in,n_out", [(1, 16, 8), (7, 48, 40), (300, 272, 520), (513, 1040, 776),
                                          (1000, 2064, 264), (3333, 3344, 4104)])
def test_fwd_dgrad_elementwise(T, n_in, n_out):
    say(f"case nvfp4w T={T} in={n_in} out={n_out}")
    q, s, t, X, dY = _nvfp4_case(T, n_in, n_out, T + n_in)
    Y, dX = _run(q, s, t, X, dY)
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_nvfp4w(X, q, s, t))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad_nvfp4w(dY, q, s, t))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e} (tensor scale {t:.3e})")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16


@pytest.mark.parametrize("cfg", range(25))
def test_tensor_scale_in_every_tile_config(tune, cfg):
    """The tensor scale is applied in each configuration's epilogue (forced through sl_set_tuning)."""
    T, n_in, n_out = 1000, 2064, 520
    say(f"case nvfp4w cfg={cfg} T={T} in={n_in} out={n_out}")
    tune(gemm=cfg)
    q, s, t, X, dY = _nvfp4_case(T, n_in, n_out, 77 + cfg)
    Y, dX = _run(q, s, t, X, dY)
    e_y = ol.rel_err(host_f64(Y), ol.linear_fwd_nvfp4w(X, q, s, t))
    e_dx = ol.rel_err(host_f64(dX), ol.linear_dgrad_nvfp4w(dY, q, s, t))
    say(f"  rel err Y {e_y:.2e} dX {e_dx:.2e}")
    assert e_y <= TOL_BF16 and e_dx <= TOL_BF16


def test_unit_tensor_scale_matches_bf16_entry_points():
    """With t = 1 the scaled products are the plain bf16 products over the materialised weight,
    bit for bit (multiplying the accumulators by 1 changes nothing)."""
    say("case nvfp4w t=1 against sl_linear_fwd / sl_linear_dgrad")
    q, s, _, X, dY = _nvfp4_case(520, 1040, 776, 5)
    Wm = sl.sl_nvfp4_materialize(dev_u8(q), dev_u8(s))
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    a, b = sl.sl_linear_fwd_nvfp4w(Xd, Wm, 1.0), sl.sl_linear_fwd(Xd, Wm)
    c, d = sl.sl_linear_dgrad_nvfp4w(dYd, Wm, 1.0), sl.sl_linear_dgrad(dYd, Wm)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


@pytest.mark.timeout(900)
def test_full_size_workload_sampled():
    """The NVFP4-weight MLP workload at full size, in the benchmark's launch order: per micro-batch
    the weight is materialised into its param_data view before each fwd and dgrad (the first
    backward layer reuses its forward's copy), and the bf16 weight gradient accumulates all 8
    micro-batches into the zeroed grad buffer.  The materialised weight is checked bit for bit, Y
    and dX on sampled rows, main_grad on sampled entries."""
    w = configs.WORKLOADS["c7"]
    names = list(w.step_params)
    buf = sl.ParamAndGradBuffer(w.params, "cuda")
    buf.zero_grad_buffer()
    rng = np.random.default_rng(7)
    st = {}
    for name in names:
        o, i = w.params[name]
        q, s, t = configs.weight(w, name)
        st[name] = dict(q=q, s=s, t=t, qd=dev_u8(q), sd=dev_u8(s), so=rng.integers(0, o, 256),
                        si=rng.integers(0, i, 256), acc=np.zeros((256, 256)))
    for k in range(w.microbatches):
        xk = {n: configs.x(w, n, k) for n in names}
        dyk = {n: configs.dy(w, n, k) for n in names}
        Ys, dXs = {}, {}
        for name in names:
            c = st[name]
            sl.sl_nvfp4_materialize(c["qd"], c["sd"], buf.param(name))
            if k == 0:
                torch.cuda.synchronize()
                assert np.array_equal(host_bits(buf.param(name)), _want_bits(c["q"], c["s"])), name
            Ys[name] = sl.sl_linear_fwd_nvfp4w(dev_bf16(xk[name]), buf.param(name), c["t"])
        for name in reversed(names):
            c = st[name]
            if name != names[-1]:
                sl.sl_nvfp4_materialize(c["qd"], c["sd"], buf.param(name))
            dYd = dev_bf16(dyk[name])
            dXs[name] = sl.sl_linear_dgrad_nvfp4w(dYd, buf.param(name), c["t"])
            sl.sl_linear_wgrad_accum(dev_bf16(xk[name]), dYd, buf.main_grad(name))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, w.tokens - 1], np.random.default_rng(k).integers(0, w.tokens, 48)]))
        for name in names:
            c = st[name]
            say(f"  c7 mb={k} {name} {w.params[name]}")
            e_y = ol.rel_err(host_f64(Ys[name])[rows], ol.linear_fwd_nvfp4w(xk[name][rows], c["q"], c["s"], c["t"]))
            e_dx = ol.rel_err(host_f64(dXs[name])[rows], ol.linear_dgrad_nvfp4w(dyk[name][rows], c["q"], c["s"], c["t"]))
            say(f"    sampled rel err Y {e_y:.2e} dX {e_dx:.2e}")
            assert e_y <= TOL_BF16 and e_dx <= TOL_BF16
            c["acc"] = ol.linear_wgrad_accum(c["acc"], xk[name][:, c["si"]], dyk[name][:, c["so"]])
    for name in names:
        c = st[name]
        got = host_f64(buf.main_grad(name))[c["so"], c["si"]]
        e = ol.rel_err(got, np.diag(c["acc"]))
        say(f"  c7 {name} main_grad sampled rel err {e:.2e}")
        assert e <= 1e-4
