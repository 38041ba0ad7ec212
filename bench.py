"""Throughput of one TP rank's linear step on one MI355X, against the MFMA roofline.

A step is one pass of the whole hot path over one batch of synthetic input: zero the fp32
grad_data once, then for every micro-batch run the forward GEMM of each weight shard, and in
backward order its dgrad and its fused fp32 wgrad-accumulate into the main_grad view.  Inputs
are resident in HBM before timing starts.  The value is algorithmic TFLOP/s (2*T*in*out per
GEMM) of K timed steps with one HIP event per step boundary; a second pass of K steps brackets
every kernel launch with HIP events on the launch stream to give the per-kernel roofline
figures (those events slow the step, so they stay out of the headline pass).

    python bench.py [--steps K] [--warmup W] [--config c2|c1|c3|c4|c5|c6|c7] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s fwd+dgrad+wgrad per TP-sharded linear; % of MI355X MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}      # MI355X published dense MFMA peaks
HBM_GBS = 8000.0
# 256 CUs x 2.4 GHz peak engine clock x 4096 bf16 (8192 fp8) dense FLOP per clock per CU
PEAK_FORMULA = {"bf16": "256 CU x 2.4 GHz x 4096 FLOP/clk/CU = 2.52 PFLOP/s (published 2.5)",
                "fp8": "256 CU x 2.4 GHz x 8192 FLOP/clk/CU = 5.03 PFLOP/s (published 5.0)"}
HIP_ATTR_CLOCK_RATE = 5     # hipDeviceAttributeClockRate in hip_runtime_api.h (peak clock, kHz)


def device_clock_mhz():
    """Peak engine clock the HIP runtime reports for device 0 (MHz), or None."""
    import ctypes
    from sharded_linear_amd import _lib
    try:
        rt = ctypes.CDLL(_lib.hip_runtimes_mapped()[0])
        v = ctypes.c_int(0)
        if rt.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_CLOCK_RATE, 0) == 0:
            return round(v.value / 1000.0, 1)
    except Exception:
        pass
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="c2")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-kernel-events", action="store_true",
                   help="skip the second pass that times every launch with HIP events")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES (reference for HBM byte counters)")
    p.add_argument("--vendor-compare", action="store_true",
                   help="only time the bf16 forward and dgrad against torch's library GEMMs on the "
                        "workload's shapes (context for the per-kernel figures; not the step)")
    return p.parse_args()


def kernel_sources_digest() -> str:
    """sha256 over the kernel sources with their comments removed, so that a comment edit does
    not void the counter records; any change to the code does."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sharded_linear_amd", "csrc", "*"))):
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
        h.update(os.path.basename(f).encode() + b"\0" + code.encode())
    return h.hexdigest()


def stored_traffic(workload_key: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter record of this
    workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is none or the kernel
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_key}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if kernel_sources_digest() != rec.get("kernel_sources_sha256"):
        return None
    b = rec.get("per_launch_bytes", {}).get(kernel)
    return None if b is None else int(b["fetch"] + b["write"])


def copy_calibration(nbytes: int) -> None:
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
    convert the counters of the GEMM kernels into HBM bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def vendor_compare(w, steps: int) -> None:
    """Context for the per-kernel figures: the library's bf16 forward and dgrad beside torch's own
    GEMMs on the same shapes (F.linear and matmul, hipBLASLt on ROCm), called in turn with the
    operands rotating over 8 sets so that no call finds its inputs in the caches of the previous
    one, HIP events around every call; one JSON line per shard with the medians.  The library
    GEMMs are timed here only; the step never calls them."""
    import torch
    import torch.nn.functional as F

    import sharded_linear_amd as sl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev).manual_seed(2024)
    sets, T = 8, w.tokens
    for n in w.step_params:
        o, i = w.params[n]
        rnd = lambda shape, std=1.0: (torch.randn(shape, device=dev, generator=gen) * std).to(torch.bfloat16)
        Xs = [rnd((T, i)) for _ in range(sets)]
        Ws = [rnd((o, i), 0.02) for _ in range(sets)]
        dYs = [rnd((T, o)) for _ in range(sets)]
        Y = torch.empty((T, o), dtype=torch.bfloat16, device=dev)
        dX = torch.empty((T, i), dtype=torch.bfloat16, device=dev)
        fns = {"fwd": lambda j: sl.sl_linear_fwd(Xs[j], Ws[j], Y),
               "fwd_library": lambda j: F.linear(Xs[j], Ws[j]),
               "dgrad": lambda j: sl.sl_linear_dgrad(dYs[j], Ws[j], dX),
               "dgrad_library": lambda j: torch.matmul(dYs[j], Ws[j])}
        for j in range(sets):
            for f in fns.values():
                f(j)
        torch.cuda.synchronize()
        ev = {k: [] for k in fns}
        for r in range(steps):
            for k, f in fns.items():
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                f(r % sets)
                e.record()
                ev[k].append((s, e))
        torch.cuda.synchronize()
        flops = 2 * T * i * o
        rec = {"vendor_compare": n, "T_in_out": [T, i, o], "calls": steps}
        for k, v in ev.items():
            us = sorted(s.elapsed_time(e) * 1e3 for s, e in v)[len(v) // 2]
            rec[k] = {"median_us": round(us, 2), "tflops": round(flops / us / 1e6, 1)}
        print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard only: run it with --gpus 1 (the library has no "
              "multi-GPU collectives)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.vendor_compare:
        from synth import configs
        vendor_compare(configs.WORKLOADS[args.config], max(args.steps, 20))
        return

    import numpy as np
    import torch

    import sharded_linear_amd as sl
    from synth import configs

    w = configs.WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def dev_u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- set-up: layout, buffers, weights, all micro-batches resident in HBM ----------------
    t0 = time.time()
    buf = sl.ParamAndGradBuffer(w.params, dev)
    names = list(w.step_params)
    wq = {}
    for n in names:
        wt = configs.weight(w, n)
        if w.mxfp8:
            wq[n] = (dev_u8(wt[0]), dev_u8(wt[1]))
        elif w.nvfp4w:
            # the NVFP4 shard (packed codes, block scales, tensor scale); the param buffer's bf16
            # view receives its materialisation once per step
            wq[n] = (dev_u8(wt[0]), dev_u8(wt[1]), wt[2])
        else:
            buf.param(n).copy_(dev_bf16(wt))
    xs, dys = [], []
    qb = {}
    if w.mxfp8_all:
        # MXFP8 copies made inside the step: W, X and dY rowwise ([r, c] codes, [r, c/32] scales) and
        # columnwise (transposed: [c, r] codes, [c, r/32] scales)
        def quant_bufs(r, c):
            u8 = dict(dtype=torch.uint8, device=dev)
            return (torch.empty((r, c), **u8), torch.empty((r, c // 32), **u8),
                    torch.empty((c, r), **u8), torch.empty((c, r // 32), **u8))
        for n in names:
            o, i = w.params[n]
            qb[n] = {"W": quant_bufs(o, i), "X": quant_bufs(w.tokens, i), "dY": quant_bufs(w.tokens, o)}
    for k in range(w.microbatches):
        xk, dyk = {}, {}
        for n in names:
            xv = configs.x(w, n, k)
            xk[n] = (dev_u8(xv[0]), dev_u8(xv[1])) if w.mxfp8 else dev_bf16(xv)
            dyk[n] = dev_bf16(configs.dy(w, n, k))
        xs.append(xk)
        dys.append(dyk)
    T = w.tokens
    ys = {n: torch.empty((T, w.params[n][0]), dtype=torch.bfloat16, device=dev) for n in names}
    dxs = {n: torch.empty((T, w.params[n][1]), dtype=torch.bfloat16, device=dev) for n in names}
    wss = {}
    for n in names:
        o, i = w.params[n]
        nb = (sl.sl_mxfp8_workspace_bytes(T, i, o) if w.mxfp8 else
              sl.sl_mxfp8_wgrad_workspace_bytes(T, i, o) if w.mxfp8_all else sl.sl_wgrad_workspace_bytes(T, i, o))
        wss[n] = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev) if nb else None
    torch.cuda.synchronize()
    log(f"set-up {time.time() - t0:.1f}s: {w.title}; grad_data {buf.numel} elements")

    # ---- one step --------------------------------------------------------------------------
    stream = torch.cuda.current_stream(dev)
    records = []        # (kind, flops, start_event, end_event) of the timed steps
    pool = []           # events created before the kernel pass, which then only records them
    counted = [0]       # launches per step, from a pass that launches nothing

    def launch(kind, flops, fn, *a, timed):
        if timed == "count":
            counted[0] += 1
        elif timed:
            s, e = pool.pop(), pool.pop()
            s.record(stream)
            fn(*a)
            e.record(stream)
            records.append((kind, flops, s, e))
        else:
            fn(*a)

    def step(timed=False):
        launch("zero", 0, sl.sl_grad_buffer_zero, buf.grad_data, timed=timed)
        if w.mxfp8_all:
            return step_mxfp8_all(timed)
        if w.nvfp4w:
            return step_nvfp4w(timed)
        for k in range(w.microbatches):
            for n in names:
                o, i = w.params[n]
                f = 2 * T * i * o
                if w.mxfp8:
                    launch("fwd", f, sl.sl_linear_fwd_mxfp8, *xs[k][n], *wq[n], ys[n], timed=timed)
                else:
                    launch("fwd", f, sl.sl_linear_fwd, xs[k][n], buf.param(n), ys[n], timed=timed)
            for n in reversed(names):
                o, i = w.params[n]
                f = 2 * T * i * o
                if w.mxfp8:
                    launch("dgrad", f, sl.sl_linear_dgrad_mxfp8w, dys[k][n], *wq[n], dxs[n], wss[n], timed=timed)
                    launch("wgrad", f, sl.sl_linear_wgrad_accum_mxfp8x, *xs[k][n], dys[k][n],
                           buf.main_grad(n), wss[n], timed=timed)
                else:
                    launch("dgrad", f, sl.sl_linear_dgrad, dys[k][n], buf.param(n), dxs[n], timed=timed)
                    launch("wgrad", f, sl.sl_linear_wgrad_accum, xs[k][n], dys[k][n], buf.main_grad(n),
                           wss[n], timed=timed)

    def step_mxfp8_all(timed):
        # weights: quantised once per step (fixed across its micro-batches), both directions
        for n in names:
            launch("quant", 0, sl.sl_mxfp8_quantize, buf.param(n), True, True, qb[n]["W"], timed=timed)
        for k in range(w.microbatches):
            for n in names:
                o, i = w.params[n]
                Xq, Xs, _, _ = qb[n]["X"]
                Wq, Ws, _, _ = qb[n]["W"]
                launch("quant", 0, sl.sl_mxfp8_quantize, xs[k][n], True, True, qb[n]["X"], timed=timed)
                launch("fwd", 2 * T * i * o, sl.sl_linear_fwd_mxfp8, Xq, Xs, Wq, Ws, ys[n], timed=timed)
            for n in reversed(names):
                o, i = w.params[n]
                dYq, dYs, dYqT, dYsT = qb[n]["dY"]
                _, _, WqT, WsT = qb[n]["W"]
                _, _, XqT, XsT = qb[n]["X"]
                launch("quant", 0, sl.sl_mxfp8_quantize, dys[k][n], True, True, qb[n]["dY"], timed=timed)
                launch("dgrad", 2 * T * i * o, sl.sl_linear_dgrad_mxfp8, dYq, dYs, WqT, WsT, dxs[n], timed=timed)
                launch("wgrad", 2 * T * i * o, sl.sl_linear_wgrad_accum_mxfp8, dYqT, dYsT, XqT, XsT,
                       buf.main_grad(n), wss[n], timed=timed)

    def step_nvfp4w(timed):
        # NVFP4 weights materialised (exact bf16 products E2M1 x E4M3) right before each fwd and
        # dgrad, which read them with the fp32 tensor scale in the epilogue: the fresh copy is still
        # in the caches when the GEMM reads it, which more than pays for the extra materialisations
        for k in range(w.microbatches):
            for n in names:
                o, i = w.params[n]
                launch("materialize", 0, sl.sl_nvfp4_materialize, wq[n][0], wq[n][1], buf.param(n), timed=timed)
                launch("fwd", 2 * T * i * o, sl.sl_linear_fwd_nvfp4w, xs[k][n], buf.param(n), wq[n][2], ys[n],
                       timed=timed)
            for n in reversed(names):
                o, i = w.params[n]
                f = 2 * T * i * o
                # the last forward layer is the first backward one: its copy from the forward is
                # unchanged (weights change only between steps) and still cache-resident
                if n != names[-1]:
                    launch("materialize", 0, sl.sl_nvfp4_materialize, wq[n][0], wq[n][1], buf.param(n), timed=timed)
                launch("dgrad", f, sl.sl_linear_dgrad_nvfp4w, dys[k][n], buf.param(n), wq[n][2], dxs[n],
                       timed=timed)
                launch("wgrad", f, sl.sl_linear_wgrad_accum, xs[k][n], dys[k][n], buf.main_grad(n), wss[n],
                       timed=timed)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Headline pass: K steps with one event per step boundary only.  Events around every launch
    # cost 4 % (config 2) to 10 % (config 3) of the step, so they get a pass of their own below.
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    bounds[0].record(stream)
    for k in range(args.steps):
        step()
        bounds[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = bounds[0].elapsed_time(bounds[-1]) / args.steps
    step_ms = sorted(bounds[k].elapsed_time(bounds[k + 1]) for k in range(args.steps))
    # Kernel pass: K more steps with HIP events around every launch on the launch stream, for the
    # per-kernel durations and the roofline figures.  The events are created beforehand and the
    # garbage collector is paused: with up to 83 launches a step, creating two events per launch
    # inside the pass slowed the host enough to let the GPU queue run dry inside some brackets.
    if not args.no_kernel_events:
        step(timed="count")
        pool.extend(torch.cuda.Event(enable_timing=True) for _ in range(2 * counted[0] * args.steps))
        gc.disable()
        try:
            for _ in range(args.steps):
                step(timed=True)
            torch.cuda.synchronize()
        finally:
            gc.enable()
    flops = w.flops_per_step()
    tflops = flops / (ms * 1e-3) / 1e12
    # MXFP8 workload: fwd runs block-scaled fp8 MFMA, dgrad/wgrad bf16 MFMA on the exactly
    # dequantised operand; the bf16 peak is the conservative denominator for the whole step.
    dtype = ("mxfp8-e4m3 fwd / bf16 bwd" if w.mxfp8 else "mxfp8-e4m3" if w.mxfp8_all else
             "bf16 (nvfp4 weights)" if w.nvfp4w else "bf16")
    peak = PEAK_TFLOPS["fp8"] if w.mxfp8_all else PEAK_TFLOPS["bf16"]
    med = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    # ---- per-kernel figures from the events -----------------------------------------------
    kinds = {}
    for kind, f, s, e in records:
        d = kinds.setdefault(kind, {"launches": 0, "ms": 0.0, "flops": 0})
        d["launches"] += 1
        d["ms"] += s.elapsed_time(e)
        d["flops"] += f
    kernels = {}
    for kind, d in kinds.items():
        avg_us = d["ms"] / d["launches"] * 1e3
        kernels[kind] = {"launches_per_step": d["launches"] // args.steps, "avg_us": round(avg_us, 2),
                         "share_of_event_pass": round(d["ms"] / sum(x["ms"] for x in kinds.values()), 4)}
        if d["flops"]:
            kernels[kind]["tflops"] = round(d["flops"] / (d["ms"] * 1e-3) / 1e12, 1)
    roofline = None
    gemm = {k: v for k, v in kinds.items() if v["flops"]}
    if gemm:
        dom = max(gemm, key=lambda k: gemm[k]["ms"])
        d = gemm[dom]
        ach = d["flops"] / (d["ms"] * 1e-3) / 1e12
        kpeak = PEAK_TFLOPS["fp8"] if ((w.mxfp8 and dom == "fwd") or w.mxfp8_all) else peak
        roofline = {"kernel": f"linear_{dom}", "bound": "mfma", "achieved": round(ach, 1), "peak": kpeak,
                    "unit": "TFLOP/s", "frac": round(ach / kpeak, 4),
                    "traffic": stored_traffic(w.key, f"linear_{dom}"),
                    "per_launch_flops": d["flops"] // d["launches"], "avg_launch_us": round(d["ms"] / d["launches"] * 1e3, 2)}

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded N(0,1) activations/grads, N(0,0.02^2) weights, bf16 RNE)",
        "config": {"workload": w.title, "key": w.key, "tokens": T, "microbatches": w.microbatches,
                   "shards_out_in": {n: list(w.params[n]) for n in names},
                   "flops_per_step": flops, "step": "zero grad_data; per micro-batch: fwd of each "
                   "shard, then dgrad + fused fp32 wgrad-accumulate in backward order" +
                   ("; W quantised once per step, X before fwd and dY before dgrad, each rowwise and "
                    "columnwise (MXFP8 quantisation kernels inside the timed step)" if w.mxfp8_all else
                    "; NVFP4 weights materialised to bf16 right before each fwd and dgrad (inside the timed "
                    "step; the first backward layer reuses its forward's copy), which are scaled by the fp32 "
                    "tensor scale" if w.nvfp4w else "")},
        "frac_of_peak": round(tflops / peak, 4),
        "step_ms": {"median": round(med, 4), "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4),
                    "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 2),
                    "tflops_at_min": round(flops / (step_ms[0] * 1e-3) / 1e12, 2)},
        "peak_formula": PEAK_FORMULA["fp8" if w.mxfp8_all else "bf16"],
        "roofline": roofline, "kernels": kernels, "cpu_baseline": cpu,
        "gpu": torch.cuda.get_device_name(dev),
        "cu_count": torch.cuda.get_device_properties(dev).multi_processor_count,
        "peak_engine_clock_mhz": device_clock_mhz(),
    }
    if w.mxfp8:
        # a third of the FLOPs (fwd) can run at the fp8 rate, two thirds (dgrad, wgrad) at bf16
        p_mix = 3.0 / (1.0 / PEAK_TFLOPS["fp8"] + 2.0 / PEAK_TFLOPS["bf16"])
        out["mxfp8_fractions"] = {
            "of_flop_mix_weighted_peak": round(tflops / p_mix, 4), "flop_mix_weighted_peak": round(p_mix, 1),
            "of_raw_fp8_peak": round(tflops / PEAK_TFLOPS["fp8"], 4),
            "per_gemm": {k: round(v["tflops"] / (PEAK_TFLOPS["fp8"] if k == "fwd" else PEAK_TFLOPS["bf16"]), 4)
                         for k, v in kernels.items() if "tflops" in v}}
    print(json.dumps(out), flush=True)


def cpu_baseline(w):
    """The oracle (numpy float64, BLAS dgemm) timed on the host over whole micro-batches of the
    same workload until about 10 s have passed."""
    import numpy as np
    from oracle import linear as ol
    from oracle import numerics
    from synth import configs

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:                       # threadpoolctl missing: report the affinity mask
        threads = 0
    cores = threads or len(os.sched_getaffinity(0))
    host = {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas_threads": threads}
    if w.mxfp8:
        log("cpu baseline: MXFP8 workload, oracle dequantises per block first")
    names = list(w.step_params)
    weights = {n: configs.weight(w, n) for n in names}
    done_flops, elapsed, mbs = 0, 0.0, 0
    if w.mxfp8_all:
        return cpu_baseline_mxfp8_all(w, names, weights, cores, host)
    if w.nvfp4w:
        log("cpu baseline: NVFP4-weight workload, oracle decodes the weight once")
        weights = {n: numerics.nvfp4_dequant(*weights[n]) for n in names}
    for k in range(w.microbatches):
        xk = {n: configs.x(w, n, k) for n in names}
        dyk = {n: configs.dy(w, n, k) for n in names}
        t = time.perf_counter()
        for n in names:
            G = np.zeros(w.params[n])
            if w.mxfp8:
                ol.linear_fwd_mxfp8(*xk[n], *weights[n])
                ol.linear_dgrad_mxfp8w(dyk[n], *weights[n])
                ol.linear_wgrad_accum_mxfp8x(G, *xk[n], dyk[n])
            else:
                ol.step(weights[n], [xk[n]], [dyk[n]], main_grad0=G)
        elapsed += time.perf_counter() - t
        done_flops += sum(6 * w.tokens * o * i for o, i in (w.params[n] for n in names))
        mbs += 1
        log(f"cpu baseline: micro-batch {k} done, {elapsed:.1f}s")
        if elapsed > 10.0:
            break
    # the single-core brute-force oracle (pure-Python triple loop) on a slice of config 1
    c1 = configs.WORKLOADS["c1"]
    rows = 4
    Xc = configs.x(c1, "weight", 0)[:rows]
    Wc = configs.weight(c1, "weight")
    t = time.perf_counter()
    ol.fwd_brute(Xc, Wc)
    tb = time.perf_counter() - t
    o1, i1 = c1.params["weight"]
    brute = {"value": round(2 * rows * i1 * o1 / tb / 1e9, 4), "unit": "GFLOP/s", "cores": 1,
             "sample": f"forward of {rows} of {c1.tokens} rows of config 1 ({o1}x{i1} weight), {tb:.2f}s"}
    return {"value": round(done_flops / elapsed / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "host": host, "brute_force_c1": brute,
            "sample": f"{mbs} of {w.microbatches} micro-batches of the same workload (fwd, dgrad, "
                      f"wgrad-accumulate of every shard), numpy float64, {elapsed:.1f}s"}


def cpu_baseline_mxfp8_all(w, names, weights, cores, host):
    """The oracle on the all-MXFP8 workload: quantisation of W (once) and of X and dY (per
    micro-batch, rowwise and columnwise) in float64, then the products over the dequantised
    values, on the first 1024 tokens of each micro-batch until about 10 s have passed."""
    import numpy as np
    from oracle import linear as ol
    from oracle import numerics
    from synth import configs

    rows = 1024
    t = time.perf_counter()
    wq = {}
    for n in names:
        wf = numerics.bf16_bits_to_f64(weights[n])
        wq[n] = (numerics.mx_quantize(wf), numerics.mx_quantize_cols(wf))
    elapsed, done_flops, mbs = time.perf_counter() - t, 0, 0
    for k in range(w.microbatches):
        xk = {n: configs.x(w, n, k)[:rows] for n in names}
        dyk = {n: configs.dy(w, n, k)[:rows] for n in names}
        t = time.perf_counter()
        for n in names:
            (wr, ws_), (wcq, wcs) = wq[n]
            xf, dyf = numerics.bf16_bits_to_f64(xk[n]), numerics.bf16_bits_to_f64(dyk[n])
            xr, xc, dr, dc = (numerics.mx_quantize(xf), numerics.mx_quantize_cols(xf),
                              numerics.mx_quantize(dyf), numerics.mx_quantize_cols(dyf))
            ol.linear_fwd_mxfp8(*xr, wr, ws_)
            ol.linear_dgrad_mxfp8(*dr, wcq, wcs)
            ol.linear_wgrad_accum_mxfp8(np.zeros(w.params[n]), *dc, *xc)
        elapsed += time.perf_counter() - t
        done_flops += sum(6 * rows * o * i for o, i in (w.params[n] for n in names))
        mbs += 1
        log(f"cpu baseline: micro-batch {k} slice done, {elapsed:.1f}s")
        if elapsed > 10.0:
            break
    return {"value": round(done_flops / elapsed / 1e12, 4), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "host": host,
            "sample": f"first {rows} of {w.tokens} tokens of {mbs} of {w.microbatches} micro-batches (weight "
                      f"quantisation once, X/dY quantisation rowwise and columnwise, fwd, dgrad, "
                      f"wgrad-accumulate of every shard), numpy float64, {elapsed:.1f}s"}


if __name__ == "__main__":
    main()
