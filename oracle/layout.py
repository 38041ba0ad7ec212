"""Reverse-order, padded layout of the contiguous param/grad buffer, as a plain Python loop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rules, all from [ATLAS-BUF] ("05 · grad/param buffer"):
  * section 4.1: parameters are placed in reverse definition order (backprop order), so offset 0
    holds the model's last parameter and bucket 0 fills first in backward;
  * section 4.2: under the distributed optimizer each parameter's start is padded up to a
    multiple of 64 *elements* (the page notes the "64-byte" docstring is wrong), and each
    bucket's end is padded to lcm(dp, 128), or lcm(dp, 128, 2^16) with the high-bus-bandwidth
    option, so every bucket splits into dp equal shards;
  * section 4.3: bucket_size counts elements, default max(40,000,000, 1,000,000 * dp); a bucket
    is closed as soon as (param_end - bucket_start) >= bucket_size, so the cut does not respect
    parameter boundaries in the sense that a bucket may run past bucket_size by one parameter;
    with bucketing disabled everything lands in one bucket;
  * section 5: both buffers are allocated zero-filled with the padded total numel; each
    parameter's weight and main_grad are views [start, end) of param_data / grad_data.
  [MEGA-SRC] section 6.3 gives the worked toy: W1(6), W2(4), WL(12) defined in that order land
  at WL [0,12), W2 [12,16), W1 [16,22), numel 22, and at dp=2 the shard boundary is element 11.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


def default_bucket_size(dp: int) -> int:
    """max(40,000,000, 1,000,000 * dp) elements ([ATLAS-BUF] section 4.3)."""
    return max(40_000_000, 1_000_000 * dp)


def bucket_divisor(dp: int, high_busbw: bool = False) -> int:
    """Bucket-end padding divisor lcm(dp, 128) or lcm(dp, 128, 2^16) ([ATLAS-BUF] section 4.2)."""
    d = dp * 128 // math.gcd(dp, 128)
    if high_busbw:
        d = d * 65536 // math.gcd(d, 65536)
    return d


def _round_up(x: int, m: int) -> int:
    return -(-x // m) * m


@dataclass
class Layout:
    start: list = field(default_factory=list)        # per parameter, definition order
    end: list = field(default_factory=list)
    bucket_id: list = field(default_factory=list)
    buckets: list = field(default_factory=list)      # (offset, numel_padded, numel_unpadded)
    numel: int = 0


def build_layout(numels, param_align: int = 64, bucket_size=None, dp: int = 1, divisor=None):
    """Place parameters (numels given in definition order) into one padded buffer.

    bucket_size None disables bucketing (one bucket).  divisor defaults to lcm(dp, 128).
    """
    if divisor is None:
        divisor = bucket_divisor(dp)
    n = len(numels)
    lay = Layout(start=[0] * n, end=[0] * n, bucket_id=[0] * n)
    bucket_start = 0
    cursor = 0
    bucket = 0
    open_params = 0
    last_end = 0
    for p in reversed(range(n)):               # backprop order
        s = _round_up(cursor, param_align)
        e = s + int(numels[p])
        lay.start[p], lay.end[p], lay.bucket_id[p] = s, e, bucket
        open_params += 1
        last_end = e
        cursor = e
        if bucket_size is not None and e - bucket_start >= bucket_size:
            padded = _round_up(e, divisor)
            lay.buckets.append((bucket_start, padded - bucket_start, e - bucket_start))
            bucket_start = cursor = padded
            bucket += 1
            open_params = 0
    if open_params:
        padded = _round_up(last_end, divisor)
        lay.buckets.append((bucket_start, padded - bucket_start, last_end - bucket_start))
        bucket_start = padded
    lay.numel = bucket_start
    return lay


def shard_ranges(bucket_offset: int, bucket_numel: int, dp: int):
    """The dp equal element ranges of one bucket; rank r owns the r-th ([ATLAS-BUF] section 6.5).
    They ignore parameter boundaries."""
    assert bucket_numel % dp == 0
    w = bucket_numel // dp
    return [(bucket_offset + r * w, bucket_offset + (r + 1) * w) for r in range(dp)]
