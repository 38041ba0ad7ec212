"""The weight gradient without allocation (sl_linear_wgrad_accum_noalloc) against the workspace
entry point sl_linear_wgrad_accum, through the C ABI.

Both run the same plan and kernels, so their main_grad must agree bit for bit; each is also held
to the fp32 bar against the oracle.  Two calls in a row on the library's scratch array, the second
with a smaller input (fewer, smaller partial planes over what the first call left there), then an
unsplit shape and a shape whose planes exceed the array.
"""
import ctypes

import numpy as np
import pytest
import torch

import sharded_linear_amd as sl
import synth
from oracle import linear as ol
from sharded_linear_amd import _lib
from tests.gpu_util import dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4


def _case(T, n_in, n_out, seed):
    X = synth.normal_bf16((T, n_in), seed)
    dY = synth.normal_bf16((T, n_out), seed + 1)
    G0 = synth.normal_f32((n_out, n_in), seed + 2)
    return X, dY, G0


def _both(T, n_in, n_out, seed):
    X, dY, G0 = _case(T, n_in, n_out, seed)
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    Ga = torch.from_numpy(G0).cuda()
    Gb = torch.from_numpy(G0).cuda()
    sl.sl_linear_wgrad_accum(Xd, dYd, Ga)
    sl.sl_linear_wgrad_accum_noalloc(Xd, dYd, Gb)
    torch.cuda.synchronize()
    return X, dY, G0, Ga, Gb


@pytest.mark.parametrize("first,second", [((8192, 2048, 1536), (2048, 1024, 1536))])
def test_noalloc_matches_workspace_entry_point(first, second):
    L = _lib.lib()
    for (T, n_in, n_out), seed in ((first, 71), (second, 81)):
        need = L.sl_wgrad_workspace_bytes(T, n_in, n_out)
        say(f"case noalloc T={T} in={n_in} out={n_out} planes={need} bytes")
        assert 0 < need <= L.sl_wgrad_workspace_bytes(*first)   # split; the second is no larger
        X, dY, G0, Ga, Gb = _both(T, n_in, n_out, seed)
        assert torch.equal(Ga.view(torch.int32), Gb.view(torch.int32))
        e = ol.rel_err(host_f64(Gb), ol.linear_wgrad_accum(G0, X, dY))
        say(f"  bitwise equal to the workspace entry point; rel err vs oracle {e:.2e}")
        assert e <= TOL_F32


def test_noalloc_unsplit_shape():
    T, n_in, n_out = 300, 520, 264                # 6 tiles, too few k stages to split
    assert _lib.lib().sl_wgrad_workspace_bytes(T, n_in, n_out) == 0
    say(f"case noalloc unsplit T={T} in={n_in} out={n_out}")
    X, dY, G0, Ga, Gb = _both(T, n_in, n_out, 91)
    assert torch.equal(Ga.view(torch.int32), Gb.view(torch.int32))
    assert ol.rel_err(host_f64(Gb), ol.linear_wgrad_accum(G0, X, dY)) <= TOL_F32


def test_noalloc_refuses_planes_beyond_the_array():
    L = _lib.lib()
    T, n_in, n_out = 8192, 4096, 1536             # 3 planes of 24 MiB
    assert L.sl_wgrad_workspace_bytes(T, n_in, n_out) > 64 << 20
    X = torch.zeros((T, n_in), dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros((T, n_out), dtype=torch.bfloat16, device="cuda")
    G = torch.ones((n_out, n_in), dtype=torch.float32, device="cuda")
    st = L.sl_linear_wgrad_accum_noalloc(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                          X.data_ptr(), dY.data_ptr(), G.data_ptr(), T, n_in, n_out)
    assert st == -4                               # SL_EWORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert bool((G == 1).all())
