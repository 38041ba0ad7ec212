"""The C++ layout builder (through the C ABI) against the oracle's layout loop."""
import numpy as np
import pytest

from oracle import layout as olayout
from sharded_linear_amd import sl_bucket_divisor, sl_default_bucket_size, sl_layout_build
from sharded_linear_amd import _lib


def same(numels, align, bs, div):
    got = sl_layout_build(numels, align, bs, div)
    ref = olayout.build_layout(numels, param_align=align, bucket_size=bs, divisor=div)
    assert got.start == ref.start and got.end == ref.end and got.bucket_id == ref.bucket_id
    assert [(b.offset, b.numel, b.numel_unpadded) for b in got.buckets] == ref.buckets
    assert got.numel == ref.numel
    return got


def test_toy():
    lay = same([6, 4, 12], 1, None, 2)
    assert lay.numel == 22 and (lay.start, lay.end) == ([16, 12, 0], [22, 16, 12])


def test_configs():
    bs = sl_default_bucket_size(1)
    same([512 * 256], 64, None, 128)
    same([8192 * 2048, 2048 * 4096], 64, bs, 128)
    same([1536 * 2048, 2048 * 1024, 8192 * 2048, 2048 * 4096], 64, bs, 128)
    lay = same([6144 * 4096, 4096 * 2048, 11008 * 4096, 4096 * 5504], 64, bs, 128)
    assert len(lay.buckets) == 2


def test_helpers_match_oracle():
    for dp in (1, 2, 3, 8, 64, 96, 1000):
        assert sl_default_bucket_size(dp) == olayout.default_bucket_size(dp)
        for hb in (False, True):
            assert sl_bucket_divisor(dp, hb) == olayout.bucket_divisor(dp, hb)
    assert sl_bucket_divisor(0) == 0


def test_7b_ledger_through_the_abi():
    dp = 64
    lay = same([1_000_000] * 1875, 64, sl_default_bucket_size(dp), sl_bucket_divisor(dp, True))
    assert len(lay.buckets) == 30


@pytest.mark.parametrize("seed", range(40))
def test_random_lists(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(0, 60))
    numels = [int(x) for x in rng.integers(0, 3000, size=n)]
    if n and seed % 3 == 0:
        numels[int(rng.integers(0, n))] = int(rng.choice([1, 63, 65, 127, 129]))
    align = int(rng.choice([1, 2, 64, 128]))
    bs = None if seed % 5 == 0 else int(rng.integers(1, 8000))
    div = int(rng.choice([1, 2, 128, 384, 65536]))
    same(numels, align, bs, div)


def test_errors_and_capacity():
    import ctypes
    L = _lib.lib()
    n = 3
    I64, I32 = ctypes.c_int64 * n, ctypes.c_int32 * n
    num, s, e, b = I64(10, 20, 30), I64(), I64(), I32()
    off, bn, bu = (ctypes.c_int64 * 1)(), (ctypes.c_int64 * 1)(), (ctypes.c_int64 * 1)()
    nb, tot = ctypes.c_int32(), ctypes.c_int64()
    st = L.sl_layout_build(n, num, 1, 15, 1, s, e, b, 1, off, bn, bu, ctypes.byref(nb), ctypes.byref(tot))
    assert st == -6 and nb.value == 3        # every param reaches bucket_size: three buckets, one slot
    assert L.sl_layout_build(n, num, 0, 15, 1, s, e, b, 1, off, bn, bu, ctypes.byref(nb), ctypes.byref(tot)) == -1
    assert L.sl_layout_build(n, num, 1, 15, 0, s, e, b, 1, off, bn, bu, ctypes.byref(nb), ctypes.byref(tot)) == -1
    bad = I64(10, -1, 30)
    assert L.sl_layout_build(n, bad, 1, 15, 1, s, e, b, 1, off, bn, bu, ctypes.byref(nb), ctypes.byref(tot)) == -1
    assert L.sl_layout_build(0, None, 64, 0, 128, None, None, None, 0, None, None, None,
                             ctypes.byref(nb), ctypes.byref(tot)) == 0 and tot.value == 0 and nb.value == 0
