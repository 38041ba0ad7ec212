"""How the step shards, checked with two CPU ranks over gloo (no GPU, no HIP call).

The library computes one rank's share; the collectives around it are outside it.  These tests run
the oracle's products on each rank's shard and the collectives the pages put around them, and check
that they reassemble the unsharded layer (llm-infra-atlas "01 · ColumnParallelLinear /
RowParallelLinear", sections 1 and 4: a column-parallel layer followed by a row-parallel one needs
one reduction of the partial outputs; the column layer's input gradient is all-reduced), and that
the grad-buffer layout the C++ builder produces at dp = 2 splits every bucket into equal per-rank
shards for the data-parallel reduction (llm-infra-atlas "05 · grad/param buffer", sections 4.2 and
6: buckets padded to lcm(dp, 128), each rank reducing its own contiguous shard).
"""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

WORLD = 2


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _tp_rank(rank, port, out):
    os.environ["MASTER_ADDR"], os.environ["MASTER_PORT"] = "127.0.0.1", str(port)
    dist.init_process_group("gloo", rank=rank, world_size=WORLD)
    try:
        from oracle import linear as ol
        rng = np.random.default_rng(123)                  # every rank draws the same full tensors
        h, f, T = 64, 96, 40
        W1 = rng.standard_normal((f, h)) * 0.02           # column-parallel: rows split over ranks
        W2 = rng.standard_normal((h, f)) * 0.02           # row-parallel: columns split over ranks
        X = rng.standard_normal((T, h))
        dY = rng.standard_normal((T, h))
        c = f // WORLD
        W1r, W2r = W1[rank * c:(rank + 1) * c], W2[:, rank * c:(rank + 1) * c]
        # forward: the column output stays local and feeds the row shard; the row output is a
        # partial sum that one all-reduce completes
        Zr = ol.linear_fwd(X, W1r)
        Yp = torch.from_numpy(ol.linear_fwd(Zr, W2r))
        dist.all_reduce(Yp)
        # backward: the row layer's dgrad is local (its slice of dZ); the column layer's dgrad is a
        # partial sum over ranks, all-reduced; each rank's wgrads are its slices
        dZr = ol.linear_dgrad(dY, W2r)
        dXp = torch.from_numpy(ol.linear_dgrad(dZr, W1r))
        dist.all_reduce(dXp)
        G1r, G2r = ol.linear_wgrad(X, dZr), ol.linear_wgrad(Zr, dY)
        gathered = [torch.zeros(c, h, dtype=torch.float64) for _ in range(WORLD)]
        dist.all_gather(gathered, torch.from_numpy(G1r))
        # the unsharded layer on every rank, for comparison
        Z, Y = ol.linear_fwd(X, W1), None
        Y = ol.linear_fwd(Z, W2)
        dZ = ol.linear_dgrad(dY, W2)
        dX = ol.linear_dgrad(dZ, W1)
        G1, G2 = ol.linear_wgrad(X, dZ), ol.linear_wgrad(Z, dY)
        ok = (np.allclose(Yp.numpy(), Y, rtol=1e-12, atol=1e-12)
              and np.allclose(dXp.numpy(), dX, rtol=1e-12, atol=1e-12)
              and np.allclose(torch.cat(gathered).numpy(), G1, rtol=1e-12, atol=1e-12)
              and np.allclose(G2r, G2[:, rank * c:(rank + 1) * c], rtol=1e-12, atol=1e-12))
        out[rank] = int(ok)
    finally:
        dist.destroy_process_group()


def _dp_rank(rank, port, out):
    os.environ["MASTER_ADDR"], os.environ["MASTER_PORT"] = "127.0.0.1", str(port)
    dist.init_process_group("gloo", rank=rank, world_size=WORLD)
    try:
        from oracle import linear as ol
        from sharded_linear_amd import sl_bucket_divisor, sl_layout_build
        # four weights of odd sizes (so parameter starts and bucket ends need padding) and a bucket
        # size that closes a bucket after the second parameter in backprop order
        shapes = [(33, 20), (7, 50), (64, 31), (5, 13)]
        layout = sl_layout_build([o * i for o, i in shapes], 64, 1500, sl_bucket_divisor(WORLD))
        ok = len(layout.buckets) >= 2
        # each rank's micro-batch gradients accumulated into its own grad_data views
        rng = np.random.default_rng(1000 + rank)
        grad = torch.zeros(layout.numel, dtype=torch.float64)
        want = []
        for j, (o, i) in enumerate(shapes):
            X, dY = rng.standard_normal((9, i)), rng.standard_normal((9, o))
            G = torch.from_numpy(ol.linear_wgrad(X, dY))
            grad[layout.start[j]:layout.end[j]] += G.reshape(-1)
            total = G.clone()
            dist.all_reduce(total)                  # what the data-parallel reduction must produce
            want.append(total)
        # per bucket: equal contiguous shards, each rank reducing its own (reduce-scatter by
        # all-reduce + slicing, which gloo offers)
        for b in layout.buckets:
            ok &= b.numel % WORLD == 0 and b.offset % 64 == 0
            shard = b.numel // WORLD
            red = grad[b.offset:b.offset + b.numel].clone()
            dist.all_reduce(red)
            mine = red[rank * shard:(rank + 1) * shard]
            # the shards, gathered back, rebuild the reduced bucket; padding stays zero
            parts = [torch.zeros(shard, dtype=torch.float64) for _ in range(WORLD)]
            dist.all_gather(parts, mine.contiguous())
            grad[b.offset:b.offset + b.numel] = torch.cat(parts)
        for j, (o, i) in enumerate(shapes):
            ok &= bool(torch.allclose(grad[layout.start[j]:layout.end[j]].reshape(o, i), want[j], rtol=1e-12, atol=1e-12))
        covered = torch.zeros(layout.numel, dtype=torch.bool)
        for s, e in zip(layout.start, layout.end):
            covered[s:e] = True
        ok &= bool((grad[~covered] == 0).all())
        out[rank] = int(ok)
    finally:
        dist.destroy_process_group()


@pytest.mark.parametrize("fn", [_tp_rank, _dp_rank], ids=["tp_column_then_row", "dp_bucket_shards"])
def test_two_ranks(fn):
    out = mp.get_context("spawn").Array("i", WORLD)
    mp.start_processes(fn, args=(_free_port(), out), nprocs=WORLD, join=True, start_method="spawn")
    assert list(out) == [1] * WORLD
