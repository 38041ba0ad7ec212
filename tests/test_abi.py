"""The C-ABI library loads, exports every declared symbol, and validates arguments on the host.

No call here reaches a kernel launch: each one fails validation (or is a zero-extent no-op)
before any HIP call, so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

from sharded_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sharded_linear.h")

SL_OK, SL_EINVAL, SL_EALIGN, SL_ESHAPE, SL_EWORKSPACE = 0, -1, -2, -3, -4
A = 1 << 20          # an aligned fake device address, never dereferenced
MIS = A + 2          # misaligned


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sl_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    L = _lib.lib()
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(_lib.PROTOTYPES), "ctypes prototypes must mirror the header"


def test_single_hip_runtime():
    _lib.lib()
    assert len(_lib.hip_runtimes_mapped()) <= 1


def test_status_strings():
    L = _lib.lib()
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert L.sl_status_str(st).decode().startswith("SL_")
    assert L.sl_status_str(12345) == b"unknown status"


@pytest.mark.parametrize("fn", ["sl_linear_fwd", "sl_linear_dgrad"])
def test_gemm_validation(fn):
    f = getattr(_lib.lib(), fn)
    assert f(None, A, A, A, 16, 12, 16) == SL_ESHAPE          # in not a multiple of 8
    assert f(None, A, A, A, 16, 16, 20) == SL_ESHAPE          # out not a multiple of 8
    assert f(None, A, A, A, -1, 16, 16) == SL_EINVAL
    assert f(None, A, A, A, 1 << 31, 16, 16) == SL_ESHAPE
    assert f(None, A, MIS, A, 16, 16, 16) == SL_EALIGN
    assert f(None, A, A, MIS, 16, 16, 16) == SL_EALIGN
    assert f(None, None, A, A, 16, 16, 16) == SL_EINVAL
    assert f(None, A, A, None, 16, 16, 16) == SL_EINVAL
    assert f(None, None, None, None, 0, 16, 16) == SL_OK       # empty: nothing to do


def test_wgrad_validation():
    f = _lib.lib().sl_linear_wgrad_accum
    assert f(None, A, A, A, 16, 12, 16, None, 0) == SL_ESHAPE
    assert f(None, MIS, A, A, 16, 16, 16, None, 0) == SL_EALIGN
    assert f(None, A, A, MIS, 16, 16, 16, None, 0) == SL_EALIGN
    assert f(None, A, None, A, 16, 16, 16, None, 0) == SL_EINVAL
    assert f(None, None, None, None, 0, 16, 16, None, 0) == SL_OK   # T = 0 leaves main_grad as is
    # a shape that needs split-K partials refuses a missing or short workspace
    T, n_in, n_out = 8192, 1024, 2048
    need = _lib.lib().sl_wgrad_workspace_bytes(T, n_in, n_out)
    assert need > 0
    assert f(None, A, A, A, T, n_in, n_out, None, 0) == SL_EWORKSPACE
    assert f(None, A, A, A, T, n_in, n_out, A, need - 256) == SL_EWORKSPACE
    assert f(None, A, A, A, T, n_in, n_out, MIS, need) == SL_EWORKSPACE
    assert _lib.lib().sl_wgrad_workspace_bytes(0, 16, 16) == 0


def test_wgrad_split_plan():
    """The planner's split choices seen through the workspace query: a full chip of 256x256
    tiles runs unsplit; half a chip of them with a full round of 256x128 tiles runs those unsplit;
    fewer tiles split K (fp32 planes [splits][out][in])."""
    ws = _lib.lib().sl_wgrad_workspace_bytes
    assert ws(8192, 2048, 8192) == 0                   # 256 tiles of 256x256
    assert ws(8192, 4096, 2048) == 0                   # 128 of 256x256, 256 of 256x128
    assert ws(1000, 4000, 2056) == 0                   # 144 / 288, ragged
    need = ws(8192, 2048, 1536)                        # 48 tiles: split
    assert need > 0 and need % (1536 * 2048 * 4) == 0 and need // (1536 * 2048 * 4) >= 2
    assert ws(8192, 1024, 2048) > 0                    # 32 tiles, 64 of 256x128: split


def test_mxfp8_validation():
    L = _lib.lib()
    assert L.sl_linear_fwd_mxfp8(None, A, A, A, A, A, 16, 48, 16) == SL_ESHAPE     # in % 32
    assert L.sl_linear_dgrad_mxfp8w(None, A, A, A, A, 16, 48, 16, None, 0) == SL_ESHAPE
    need = L.sl_mxfp8_workspace_bytes(8192, 2048, 8192)
    assert need >= 8192 * 2048 * 2                                           # dequantised operand
    assert L.sl_linear_dgrad_mxfp8w(None, A, A, A, A, 8192, 2048, 8192, None, 0) == SL_EWORKSPACE
    assert L.sl_linear_wgrad_accum_mxfp8x(None, A, A, A, A, 8192, 2048, 8192, A, 1024) == SL_EWORKSPACE
    assert L.sl_mxfp8_workspace_bytes(0, 64, 64) == 0 and L.sl_mxfp8_workspace_bytes(8, 48, 8) == 0
    assert L.sl_linear_wgrad_accum_mxfp8x(None, A, A, A, A, 16, 48, 16, None, 0) == SL_ESHAPE
    assert L.sl_linear_fwd_mxfp8(None, A, None, A, A, A, 16, 64, 16) == SL_EINVAL   # no scales
    assert L.sl_linear_fwd_mxfp8(None, MIS, A, A, A, A, 16, 64, 16) == SL_EALIGN
    assert L.sl_linear_wgrad_accum_mxfp8x(None, A, A, A, None, 16, 64, 16, None, 0) == SL_EINVAL
    assert L.sl_linear_fwd_mxfp8(None, None, None, None, None, None, 0, 64, 16) == SL_OK


def test_all_mxfp8_validation():
    """Argument checks of the quantiser and the both-MXFP8 dgrad / wgrad, host side only."""
    L = _lib.lib()
    q = L.sl_mxfp8_quantize
    assert q(None, A, 64, 48, A, A, None, None) == SL_ESHAPE                      # cols % 32 (rows copy)
    assert q(None, A, 48, 64, None, None, A, A) == SL_ESHAPE                      # rows % 32 (cols copy)
    assert q(None, A, 64, 12, None, None, A, A) == SL_ESHAPE                      # cols % 8 (cols copy)
    assert q(None, A, 64, 64, A, None, None, None) == SL_EINVAL                   # codes without scales
    assert q(None, A, 64, 64, None, None, None, A) == SL_EINVAL
    assert q(None, None, 64, 64, A, A, None, None) == SL_EINVAL
    assert q(None, MIS, 64, 64, A, A, None, None) == SL_EALIGN
    assert q(None, A, 64, 64, None, None, MIS, A) == SL_EALIGN
    assert q(None, A, -1, 64, A, A, None, None) == SL_EINVAL
    assert q(None, None, 0, 64, None, None, None, None) == SL_OK
    d = L.sl_linear_dgrad_mxfp8
    assert d(None, A, A, A, A, A, 16, 64, 96) == SL_ESHAPE                        # out % 128
    assert d(None, A, A, A, None, A, 16, 64, 128) == SL_EINVAL
    assert d(None, MIS, A, A, A, A, 16, 64, 128) == SL_EALIGN
    w = L.sl_linear_wgrad_accum_mxfp8
    assert w(None, A, A, A, A, A, 96, 64, 64, None, 0) == SL_ESHAPE               # T % 128
    assert w(None, A, A, None, A, A, 128, 64, 64, None, 0) == SL_EINVAL
    assert w(None, A, A, A, A, MIS, 128, 64, 64, None, 0) == SL_EALIGN
    need = L.sl_mxfp8_wgrad_workspace_bytes(8192, 2048, 1536)                   # 48 tiles: split
    assert need >= 2 * 1536 * 2048 * 4
    assert w(None, A, A, A, A, A, 8192, 2048, 1536, None, 0) == SL_EWORKSPACE
    assert w(None, A, A, A, A, A, 8192, 2048, 1536, A, need - 256) == SL_EWORKSPACE
    assert L.sl_mxfp8_wgrad_workspace_bytes(8192, 2048, 8192) == 0              # 256 tiles: unsplit
    assert L.sl_mxfp8_wgrad_workspace_bytes(8192, 4096, 2048) == 0              # 128 / 256 of 256x128: unsplit
    assert L.sl_mxfp8_wgrad_workspace_bytes(100, 64, 64) == 0
    # code operands of 2 GiB or more are beyond the direct loads of the both-MXFP8 kernels
    assert d(None, A, A, A, A, A, 1 << 20, 128, 4096) == SL_ESHAPE               # dYq 4 GiB
    assert w(None, A, A, A, A, A, 1 << 20, 64, 4096, None, 0) == SL_ESHAPE       # dYqT 4 GiB


def test_nvfp4_validation():
    """Argument checks of the NVFP4 materialiser and the scaled bf16 products, host side only."""
    L = _lib.lib()
    m = L.sl_nvfp4_materialize
    assert m(None, A, A, A, 64, 24) == SL_ESHAPE                                  # cols % 16
    assert m(None, A, A, A, -1, 32) == SL_EINVAL
    assert m(None, None, A, A, 64, 32) == SL_EINVAL
    assert m(None, A, None, A, 64, 32) == SL_EINVAL
    assert m(None, MIS, A, A, 64, 32) == SL_EALIGN
    assert m(None, A, A, MIS, 64, 32) == SL_EALIGN
    assert m(None, None, None, None, 0, 32) == SL_OK
    assert m(None, None, None, None, 64, 0) == SL_OK
    for f in (L.sl_linear_fwd_nvfp4w, L.sl_linear_dgrad_nvfp4w):
        assert f(None, A, A, float("nan"), A, 16, 64, 64) == SL_EINVAL
        assert f(None, A, A, float("inf"), A, 16, 64, 64) == SL_EINVAL
        assert f(None, A, A, 1.0, A, 16, 40, 64) == SL_ESHAPE                     # in % 16
        assert f(None, A, A, 1.0, A, 16, 64, 12) == SL_ESHAPE                     # out % 8
        assert f(None, MIS, A, 1.0, A, 16, 64, 64) == SL_EALIGN
        assert f(None, A, None, 1.0, A, 16, 64, 64) == SL_EINVAL
        assert f(None, None, None, 1.0, None, 0, 64, 64) == SL_OK


def test_mxfp8_dequantize_validation():
    d = _lib.lib().sl_mxfp8_dequantize
    assert d(None, A, A, A, 64, 48) == SL_ESHAPE                                  # cols % 32
    assert d(None, A, A, A, -1, 64) == SL_EINVAL
    assert d(None, None, A, A, 64, 64) == SL_EINVAL
    assert d(None, A, None, A, 64, 64) == SL_EINVAL
    assert d(None, MIS, A, A, 64, 64) == SL_EALIGN
    assert d(None, A, A, MIS, 64, 64) == SL_EALIGN
    assert d(None, None, None, None, 0, 64) == SL_OK


def test_zero_fill_validation():
    L = _lib.lib()
    assert L.sl_grad_buffer_zero(None, A, -1) == SL_EINVAL
    assert L.sl_grad_buffer_zero(None, None, 10) == SL_EINVAL
    assert L.sl_grad_buffer_zero(None, MIS, 10) == SL_EALIGN
    assert L.sl_grad_buffer_zero(None, None, 0) == SL_OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    from sharded_linear_amd import sl_linear_fwd
    with pytest.raises(ValueError):
        sl_linear_fwd(torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(8, 8, dtype=torch.bfloat16))


def test_tuning_knobs_and_workspace_query_agree():
    """A forced split count or tile configuration changes the workspace query and the call's check
    alike (the call refuses the default-sized workspace under a forced larger split), and -1
    restores the built-in choices; unknown knobs and out-of-range values are refused."""
    L = _lib.lib()
    ws = L.sl_wgrad_workspace_bytes
    f = L.sl_linear_wgrad_accum
    T, n_in, n_out = 8192, 2048, 1536                  # 48 tiles of 256x256: split by default
    plane = n_in * n_out * 4
    default = ws(T, n_in, n_out)
    assert default > 0 and default % plane == 0
    prev = ctypes.c_int32(99)
    try:
        assert L.sl_set_tuning(3, 7, ctypes.byref(prev)) == SL_OK and prev.value == -1
        assert ws(T, n_in, n_out) == 7 * plane
        assert f(None, A, A, A, T, n_in, n_out, A, default) == SL_EWORKSPACE     # sized for the default
        assert L.sl_set_tuning(3, 1, None) == SL_OK
        assert ws(T, n_in, n_out) == 0                                             # forced unsplit
        assert L.sl_set_tuning(3, -1, ctypes.byref(prev)) == SL_OK and prev.value == 1
        assert ws(T, n_in, n_out) == default
        # a forced 256x128 configuration (cfg 20) changes the weight gradient's tile count
        assert L.sl_set_tuning(2, 20, None) == SL_OK
        forced = ws(T, n_in, n_out)
        assert forced % plane == 0 and forced != default
        assert L.sl_set_tuning(2, -1, None) == SL_OK
        assert ws(T, n_in, n_out) == default
        # validation: knob range and value ranges; a refused call changes nothing
        assert L.sl_set_tuning(5, 0, None) == SL_EINVAL and L.sl_set_tuning(-1, 0, None) == SL_EINVAL
        assert L.sl_set_tuning(0, 26, None) == SL_EINVAL and L.sl_set_tuning(3, 0, None) == SL_EINVAL
        # the 256x192 configuration is the forward's only
        assert L.sl_set_tuning(1, 25, None) == SL_EINVAL and L.sl_set_tuning(2, 25, None) == SL_EINVAL
        assert L.sl_set_tuning(0, 25, None) == SL_OK and L.sl_set_tuning(0, -1, None) == SL_OK
        assert L.sl_set_tuning(3, 65, None) == SL_EINVAL and L.sl_set_tuning(4, 3, None) == SL_EINVAL
        assert L.sl_set_tuning(4, -2, None) == SL_EINVAL
        assert ws(T, n_in, n_out) == default
    finally:
        for k in range(5):
            L.sl_set_tuning(k, -1, None)


def test_tuning_environment_variables_are_not_read(monkeypatch):
    """The library reads no environment variables: the old tuning names change nothing."""
    ws = _lib.lib().sl_wgrad_workspace_bytes
    default = ws(8192, 2048, 1536)
    for name, val in (("SL_SPLITK", "7"), ("SL_GEMM_CONFIG", "20"), ("SL_F8_CONFIG", "1")):
        monkeypatch.setenv(name, val)
    assert ws(8192, 2048, 1536) == default


def test_mxfp8x_checks_the_whole_workspace_before_launching():
    """The dequantised-X wgrad checks dequantised operand + split planes before its first launch:
    a workspace that holds only the dequantised X is refused on a split shape."""
    L = _lib.lib()
    T, n_in, n_out = 8192, 2048, 1536
    xb = (T * n_in * 2 + 255) // 256 * 256
    need = L.sl_mxfp8_workspace_bytes(T, n_in, n_out)
    assert need > xb                                          # the planes follow the operand
    assert L.sl_linear_wgrad_accum_mxfp8x(None, A, A, A, A, T, n_in, n_out, A, xb) == SL_EWORKSPACE
    assert L.sl_linear_wgrad_accum_mxfp8x(None, A, A, A, A, T, n_in, n_out, A, need - 256) == SL_EWORKSPACE


def test_noalloc_wgrad_validation():
    """The no-allocation weight gradient validates like the workspace form and refuses plans whose
    partial planes exceed its 64 MiB array, before any HIP call."""
    f = _lib.lib().sl_linear_wgrad_accum_noalloc
    ws = _lib.lib().sl_wgrad_workspace_bytes
    assert f(None, A, A, A, 16, 12, 16) == SL_ESHAPE
    assert f(None, MIS, A, A, 16, 16, 16) == SL_EALIGN
    assert f(None, A, None, A, 16, 16, 16) == SL_EINVAL
    assert f(None, A, A, A, -1, 16, 16) == SL_EINVAL
    assert f(None, None, None, None, 0, 16, 16) == SL_OK
    assert ws(8192, 4096, 1536) > 64 << 20
    assert f(None, A, A, A, 8192, 4096, 1536) == SL_EWORKSPACE
    assert 0 < ws(8192, 2048, 1536) <= 64 << 20 and 0 < ws(8192, 1024, 2048) <= 64 << 20   # c3's splits fit
