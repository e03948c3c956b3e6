#!/usr/bin/env python3
"""RMSNorm-for-training throughput on one MI355X: fwd + bwd effective HBM GB/s.

A step is one pass of the whole path over one batch: the forward
(x -> y, rstd) and the deterministic backward (dy, x, rstd -> dx, dw) of the
RMSNorm workload x[T=4096, H=4096] BF16 with a BF16 weight (the workload the
metric is quoted on; pass --config for the others). Inputs are seeded
synthetic tensors already resident in HBM. Consecutive steps rotate over
enough buffer sets (>= 1 GiB in the cycle) that no step finds its tensors in
the 256 MB Infinity Cache, so the figure is an HBM figure.

--norm layernorm times LayerNorm instead (the other normalisation of the
benchmark_normalization table on the TE page; its workloads are named
ln_T<tokens>_H<hidden>_<weight dtype>, default ln_T8192_H4096_bf16w): a step
is its forward (y, mean, rstd) and deterministic backward (dx, dgamma,
dbeta); ops fwd+bwd, fwd, bwd and 2xfwd+bwd.

--op picks what a step is (the pages time fwd, bwd and "2xfwd+bwd", the
checkpointed step: forward, forward recompute, backward):
  fwd+bwd (default)    forward, backward
  fwd | bwd            one of them (the backward reads the rstd and h that
                       a forward left in the same buffer set beforehand)
  2xfwd+bwd            forward, forward again (recompute), backward
  fwd+bwd_recompute    forward, then the backward that recomputes rstd from
                       x itself (plain forms): the checkpointed step with the
                       recompute forward folded into the backward

Timing:
* value: K steps captured in one HIP graph (the pages time graph replays),
  replayed --replays times, each between two synchronisations; the median
  replay gives ms_per_step; GB/s of algorithmic bytes.
* roofline: the same K steps launched eagerly with the library's per-kernel
  HIP-event timers on the launch stream; the dominant kernel is the
  backward row kernel (the forward for --op fwd); achieved = its
  algorithmic bytes per launch / its mean event-timed duration; peak 8 TB/s.
* cpu_baseline: the FP64 oracle on the same work, called on row slices from
  a pool of host threads (the oracle's C code runs without the interpreter
  lock), and single-threaded beside it.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "RMSNorm fwd+bwd effective HBM GB/s and % of 8 TB/s peak, per (T,H)"
DEFAULT_CONFIG = "c2_T4096_H4096_bf16w"
DEFAULT_LN_CONFIG = "ln_T8192_H4096_bf16w"
OPS = ("fwd+bwd", "fwd", "bwd", "2xfwd+bwd", "fwd+bwd_recompute")


def algorithmic_bytes(rows: int, H: int, sw: int, residual: bool, with_dres: bool):
    """Bytes the path must move (per launch): see the design doc, measurement."""
    e = rows * H
    fwd = (8 if residual else 4) * e + 4 * rows + H * sw
    bwd_row = ((8 if with_dres else 6) if residual else 6) * e + 4 * rows + H * sw
    bwd = bwd_row + 4 * H
    return fwd, bwd_row, bwd


def ln_algorithmic_bytes(rows: int, H: int, sw: int):
    """LayerNorm bytes per launch: forward reads x, gamma, beta and writes y,
    mean, rstd; the backward row kernel reads dy, x, mean, rstd, gamma and
    writes dx; the reduce writes dgamma and dbeta."""
    e = rows * H
    fwd = 4 * e + 8 * rows + 2 * H * sw
    bwd_row = 6 * e + 8 * rows + H * sw
    return fwd, bwd_row, bwd_row + 8 * H


def time_steps(args, torch, rn, _lib, dev, sets, fwd, step, n_fwd, has_bwd, bwd_keys,
               step_bytes, fwd_b, bwd_row_b, bwd_b):
    """Graph-replay and per-kernel timing of K steps (shared by both norms)."""
    import ctypes as _ct
    P = _ct.c_void_p
    n_sets = len(sets)
    K, W = args.steps, args.warmup
    cur = torch.cuda.current_stream(dev)
    sp = P(cur.cuda_stream)

    # every set gets a forward's rstd (and h) first, so a backward-only step
    # has its inputs; then the eager warm-up and a reference result for set 0
    for s in sets:
        fwd(s, sp)
    for i in range(W):
        step(sets[i % n_sets], 1, sp)
    torch.cuda.synchronize()
    out_keys = (["y"] if n_fwd else []) + (list(bwd_keys) if has_bwd else [])
    ref = {k: sets[0][k].clone() for k in out_keys}

    def capture(det: int):
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream(device=dev)
        cs.wait_stream(cur)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                csp = P(torch.cuda.current_stream(dev).cuda_stream)
                for i in range(K):
                    step(sets[i % n_sets], det, csp)
        torch.cuda.synchronize()
        return g

    def same_bits(a, b):
        return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))

    def timed_replays(g, check: bool):
        """Median wall and GPU ms of --replays replays; every replay of the
        deterministic graph must reproduce the eager result bit for bit."""
        g.replay()  # warm
        torch.cuda.synchronize()
        walls, gpus = [], []
        for _ in range(max(1, args.replays)):
            for k in out_keys:
                sets[0][k].zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t0) * 1e3)
            gpus.append(e0.elapsed_time(e1))
            if check:
                for k in out_keys:
                    assert same_bits(sets[0][k], ref[k]), f"graph {k} != eager"
        walls.sort()
        gpus.sort()
        return walls, gpus

    g_det = capture(1)
    walls, gpus = timed_replays(g_det, check=True)
    del g_det
    walls_nd = None
    if has_bwd:
        g_nd = capture(0)
        walls_nd, _ = timed_replays(g_nd, check=False)
        del g_nd

    def median(v):
        n = len(v)
        return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])

    wall_ms, gpu_ms = median(walls), median(gpus)
    ms_per_step = wall_ms / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # Per-kernel HIP-event timing of the same K steps, launched eagerly. The
    # GPU is first parked on a sleep kernel so that the host queues all K
    # steps before any runs: the kernels then run back to back and each
    # event pair brackets GPU time only, not host launch gaps.
    rn.rmsnorm_timing_read()
    rn.rmsnorm_timing_enable(True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    t0 = time.perf_counter()
    for i in range(K):
        step(sets[i % n_sets], 1, sp)
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    timers = rn.rmsnorm_timing_read()
    rn.rmsnorm_timing_enable(False)

    def avg_us(idx):
        n, ms = timers[idx]
        return (ms / n * 1e3) if n else None

    fwd_us = avg_us(_lib.RMSN_TIMER_FWD)
    bwd_row_us = avg_us(_lib.RMSN_TIMER_BWD_ROW)
    reduce_us = avg_us(_lib.RMSN_TIMER_DW_REDUCE)
    small_us = avg_us(_lib.RMSN_TIMER_BWD_SMALL)
    if not has_bwd:
        dom_name, dom_us, dom_bytes = "fwd", fwd_us, fwd_b
    elif bwd_row_us is not None:
        dom_name, dom_us, dom_bytes = "bwd_row", bwd_row_us, bwd_row_b
    else:
        dom_name, dom_us, dom_bytes = "bwd_small", small_us, bwd_b
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    fwd_gbps = fwd_b / (fwd_us * 1e-6) / 1e9 if fwd_us else None
    bwd_us = (bwd_row_us or 0.0) + (reduce_us or 0.0) if bwd_row_us else small_us
    bwd_gbps = bwd_b / (bwd_us * 1e-6) / 1e9 if bwd_us else None

    return dict(fwd_us=fwd_us, bwd_row_us=bwd_row_us, reduce_us=reduce_us, small_us=small_us,
                dom_name=dom_name, dom_bytes=dom_bytes, achieved=achieved, ms_per_step=ms_per_step,
                value=value, walls=walls, walls_nd=walls_nd, gpu_ms=gpu_ms, t_issue=t_issue, K=K,
                W=W, median=median, fwd_gbps=fwd_gbps, bwd_gbps=bwd_gbps)


def cpu_baseline(args, rows, step_bytes, op, oracle_rows):
    """Time the unchanged oracle on the whole workload: called on row slices
    from a pool of host threads, then single-threaded, each for >= --cpu-seconds."""
    def run(threads):
        bounds = [(rows * i // threads, rows * (i + 1) // threads) for i in range(threads)]
        reps = 0
        t_start = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            while True:
                list(ex.map(lambda b: oracle_rows(*b), bounds))
                reps += 1
                el = time.perf_counter() - t_start
                if el >= args.cpu_seconds:
                    return reps, el

    threads = args.cpu_threads or min(16, os.cpu_count() or 1)
    reps_n, el_n = run(threads)
    reps_1, el_1 = run(1)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(step_bytes * reps_n / el_n / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full {args.config} workload ({op}, FP64 oracle), {reps_n} repetition(s) "
                      f"in {el_n:.1f} s, rows split over {threads} host threads of "
                      f"{model or platform.processor()}",
            "single_thread": {"value": round(step_bytes * reps_1 / el_1 / 1e9, 4), "cores": 1,
                              "sample": f"{reps_1} repetition(s) in {el_1:.1f} s"}}


def result_line(args, metric, op, value, t, step_bytes, config, traffic, cpu, route=None):
    K = t["K"]
    walls, walls_nd, median = t["walls"], t["walls_nd"], t["median"]
    return {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": t["W"],
        "ms_per_step": round(t["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: FP32 row math with FP64 sums (rstd, dw); BF16 and the
        # weight dtype are storage only
        "dtype": "f32",
        "io_dtype": "bf16 activations and gradients, weight as configured",
        "data": "synthetic",
        "config": config,
        "replay_ms_per_step": {"median": round(t["ms_per_step"], 5), "min": round(walls[0] / K, 5),
                               "max": round(walls[-1] / K, 5), "replays": len(walls)},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "fwd_GBps": round(t["fwd_gbps"], 1) if t["fwd_gbps"] else None,
        "bwd_GBps": round(t["bwd_gbps"], 1) if t["bwd_gbps"] else None,
        "nondeterministic": ({"ms_per_step": round(median(walls_nd) / K, 5),
                              "value": round(step_bytes / (median(walls_nd) / K * 1e-3) / 1e9, 2)}
                             if walls_nd else None),
        "kernel_us": {"fwd": t["fwd_us"], "bwd_row": t["bwd_row_us"], "dw_reduce": t["reduce_us"],
                      "bwd_small": t["small_us"]},
        "graph_gpu_ms": round(t["gpu_ms"], 4),
        "eager_host_issue_ms_per_step": round(t["t_issue"] * 1e3 / K, 5),
        "roofline": {"bound": "hbm", "kernel": t["dom_name"], "achieved": round(t["achieved"], 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(t["achieved"] / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": t["dom_bytes"]},
        "cpu_baseline": cpu,
        "route": route,
    }


def bench_layernorm(args, np, torch, rn, _lib, lib, synth, dev, d16) -> int:
    P = ctypes.c_void_p
    op = args.op
    if op not in ("fwd+bwd", "fwd", "bwd", "2xfwd+bwd"):
        print("--norm layernorm takes --op fwd+bwd, fwd, bwd or 2xfwd+bwd", file=sys.stderr)
        return 2
    if args.config is None:
        args.config = DEFAULT_LN_CONFIG
    wl = synth.ln_config(args.config, seed=args.seed)
    T, H = wl.T, wl.H
    sw = 2 if wl.gamma.dtype == "bf16" else 4
    wdt = _lib.RMSN_BF16 if sw == 2 else _lib.RMSN_F32
    fwd_b, bwd_row_b, bwd_b = ln_algorithmic_bytes(T, H, sw)
    n_fwd = {"fwd+bwd": 1, "fwd": 1, "bwd": 0, "2xfwd+bwd": 2}[op]
    has_bwd = op != "fwd"
    step_bytes = n_fwd * fwd_b + (bwd_b if has_bwd else 0)

    def wdev(wt):
        return d16(wt.bits) if wt.dtype == "bf16" else torch.from_numpy(wt.f32.copy()).to(dev)

    gam, bet = wdev(wl.gamma), wdev(wl.beta)
    x0, dy0 = d16(wl.x), d16(wl.dy)
    per_set = 4 * T * H * 2
    n_sets = int(min(16, max(2, math.ceil((1 << 30) / per_set))))
    sets = []
    for _ in range(n_sets):
        sets.append(dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty_like(x0), dx=torch.empty_like(x0),
                         mean=torch.empty(T, dtype=torch.float32, device=dev),
                         rstd=torch.empty(T, dtype=torch.float32, device=dev),
                         dg=torch.empty(H, dtype=torch.float32, device=dev),
                         db=torch.empty(H, dtype=torch.float32, device=dev)))
    del x0, dy0
    ws = {}
    for det in (0, 1):
        nb = max(lib.layernorm_bwd_workspace_bytes(T, H, wdt, det), 256)
        raw = torch.empty(nb + 256, dtype=torch.uint8, device=dev)
        ws[det] = (raw, P(raw.data_ptr() + (-raw.data_ptr()) % 256), nb)
    eps = ctypes.c_float(wl.eps)

    def fwd(s, stream):
        _lib.check(lib.layernorm_fwd(P(s["x"].data_ptr()), P(gam.data_ptr()), P(bet.data_ptr()), wdt,
                                     eps, P(s["y"].data_ptr()), P(s["mean"].data_ptr()),
                                     P(s["rstd"].data_ptr()), T, H, stream))

    def bwd(s, det, stream):
        _, wsp, nb = ws[det]
        _lib.check(lib.layernorm_bwd(P(s["dy"].data_ptr()), P(s["x"].data_ptr()),
                                     P(s["mean"].data_ptr()), P(s["rstd"].data_ptr()),
                                     P(gam.data_ptr()), wdt, det, P(s["dx"].data_ptr()),
                                     P(s["dg"].data_ptr()), P(s["db"].data_ptr()), T, H, wsp, nb,
                                     stream))

    def step(s, det, stream):
        for _ in range(n_fwd):
            fwd(s, stream)
        if has_bwd:
            bwd(s, det, stream)

    t = time_steps(args, torch, rn, _lib, dev, sets, fwd, step, n_fwd, has_bwd, ["dx", "dg", "db"],
                   step_bytes, fwd_b, bwd_row_b, bwd_b)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        g64, b64 = wl.gamma.f64, wl.beta.f64
        mu_all, rs_all, _ = oracle.ln_fwd(wl.x, g64, b64, wl.eps, want_y=False)

        def oracle_rows(lo, hi):
            mu, rs = mu_all[lo:hi], rs_all[lo:hi]
            for _ in range(n_fwd):
                mu, rs, _ = oracle.ln_fwd(wl.x[lo:hi], g64, b64, wl.eps)
            if has_bwd:
                oracle.ln_bwd(wl.dy[lo:hi], wl.x[lo:hi], mu, rs, g64)

        cpu = cpu_baseline(args, T, step_bytes, op, oracle_rows)
    config = {"workload": args.config, "norm": "layernorm", "op": op, "T": T, "H": H,
              "w_dtype": wl.gamma.dtype, "deterministic": True, "global_batch": T, "seq_len": T,
              "parallelism": "none (1 GPU)", "buffer_sets": n_sets}
    traffic = None
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(tr_path) and op == "fwd+bwd":
        from bwd_rmsnorm_fwd_02_amd import build as _b
        rec = json.load(open(tr_path))
        if rec.get("source_hash") == _b.source_hash() and t["dom_name"] in rec.get("kernels", {}):
            traffic = rec["kernels"][t["dom_name"]]["bytes_per_launch"]
    wt = torch.bfloat16 if wl.gamma.dtype == "bf16" else torch.float32
    route = {"fwd": rn.rmsnorm_route_query("ln_fwd", T, H, wt),
             "bwd": rn.rmsnorm_route_query("ln_bwd", T, H, wt)}
    out = result_line(args, f"LayerNorm {op} effective HBM GB/s, per (T,H)", op, t["value"], t,
                      step_bytes, config, traffic, cpu, route)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--norm", choices=("rmsnorm", "layernorm"), default="rmsnorm")
    ap.add_argument("--config", default=None)
    ap.add_argument("--op", choices=OPS, default="fwd+bwd")
    ap.add_argument("--replays", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work for each of the two CPU runs")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle run (0: min(16, CPUs))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 10 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this RMSNorm path has no multi-GPU step "
              "(rows shard across GPUs with no exchange but one dw all-reduce, which is "
              "not built); run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bwd_rmsnorm_fwd_02_amd as rn
    from bwd_rmsnorm_fwd_02_amd import _lib
    from tests import synth

    lib = _lib.load()  # raises if the HIP library is missing: no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 2, "launches": 10}), flush=True)
        return 0

    P = ctypes.c_void_p
    op = args.op

    def d16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.norm == "layernorm":
        return bench_layernorm(args, np, torch, rn, _lib, lib, synth, dev, d16)
    if args.config is None:
        args.config = DEFAULT_CONFIG
    wl = synth.config(args.config, seed=args.seed)
    rows, H, T, heads = wl.rows, wl.H, wl.T, wl.heads
    residual = wl.r is not None
    with_dres = wl.dres is not None
    sw = 2 if wl.w.dtype == "bf16" else 4
    wdt = _lib.RMSN_BF16 if wl.w.dtype == "bf16" else _lib.RMSN_F32
    fwd_b, bwd_row_b, bwd_b = algorithmic_bytes(rows, H, sw, residual, with_dres)
    rc = op == "fwd+bwd_recompute"
    if rc and residual:
        print("--op fwd+bwd_recompute covers the plain and per-head forms only", file=sys.stderr)
        return 2
    if rc:  # the recompute backward reads no rstd
        bwd_row_b -= 4 * rows
        bwd_b -= 4 * rows
    n_fwd = {"fwd+bwd": 1, "fwd": 1, "bwd": 0, "2xfwd+bwd": 2, "fwd+bwd_recompute": 1}[op]
    has_bwd = op != "fwd"
    step_bytes = n_fwd * fwd_b + (bwd_b if has_bwd else 0)

    w = d16(wl.w.bits) if wl.w.dtype == "bf16" else torch.from_numpy(wl.w.f32.copy()).to(dev)
    x0 = d16(wl.xbuf if wl.xbuf is not None else wl.x)
    dy0 = d16(wl.dy)
    r0 = d16(wl.r) if residual else None
    dres0 = d16(wl.dres) if with_dres else None

    # buffer sets: the whole cycle spans >= 1 GiB so steps run from HBM
    per_set = x0.numel() * 2 + dy0.numel() * 2 + 2 * rows * H * 2 * (2 if residual else 1)
    n_sets = int(min(16, max(2, math.ceil((1 << 30) / per_set))))
    sets = []
    for i in range(n_sets):
        s = dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty(rows, H, dtype=torch.bfloat16, device=dev),
                 # the strided form's gap columns are never written: zero them so
                 # the replay check (which zeroes outputs first) sees the same gap
                 dx=torch.zeros_like(x0) if wl.xbuf is not None else torch.empty(rows, H, dtype=torch.bfloat16, device=dev),
                 rstd=torch.empty(rows, dtype=torch.float32, device=dev),
                 dw=torch.empty(H, dtype=torch.float32, device=dev))
        if residual:
            s["r"] = r0.clone()
            s["h"] = torch.empty(rows, H, dtype=torch.bfloat16, device=dev)
            s["dres"] = dres0.clone() if with_dres else None
        sets.append(s)
    del x0, dy0, r0, dres0

    # separate workspaces: the deterministic partials, and the zero-filled
    # accumulator the non-deterministic kernels keep zero-filled
    ws_bytes_det = max(lib.rmsnorm_bwd_workspace_bytes(rows, H, wdt, 1), 256)
    ws_bytes_nd = max(lib.rmsnorm_bwd_workspace_bytes(rows, H, wdt, 0), 256)
    ws_det_raw = torch.empty(ws_bytes_det + 256, dtype=torch.uint8, device=dev)
    ws_nd_raw = torch.zeros(ws_bytes_nd + 256, dtype=torch.uint8, device=dev)
    ws_det = ws_det_raw[(-ws_det_raw.data_ptr()) % 256:]
    ws_nd = ws_nd_raw[(-ws_nd_raw.data_ptr()) % 256:]
    ws_arg = {1: (P(ws_det.data_ptr()), ws_bytes_det), 0: (P(ws_nd.data_ptr()), ws_bytes_nd)}

    if wl.xbuf is not None:
        xv = _lib.View(T, heads, H, wl.x_stride_t, wl.x_stride_h)
    else:
        xv = _lib.View(T, heads, H, heads * H, H)
    cv = _lib.View(T, heads, H, heads * H, H)

    dxv = xv if wl.xbuf is not None else cv

    def fwd(s, stream):
        if residual:
            _lib.check(lib.rmsnorm_residual_fwd(P(s["x"].data_ptr()), P(s["r"].data_ptr()),
                                                P(w.data_ptr()), wdt, ctypes.c_float(wl.eps),
                                                P(s["h"].data_ptr()), P(s["y"].data_ptr()),
                                                P(s["rstd"].data_ptr()), rows, H, stream))
        else:
            _lib.check(lib.rmsnorm_fwd_strided(P(s["x"].data_ptr()), xv, P(w.data_ptr()), wdt,
                                               ctypes.c_float(wl.eps), P(s["y"].data_ptr()), cv,
                                               P(s["rstd"].data_ptr()), stream))

    def bwd(s, det: int, stream):
        wsp, ws_bytes = ws_arg[det]
        if residual:
            _lib.check(lib.rmsnorm_residual_bwd(P(s["dy"].data_ptr()), P(s["h"].data_ptr()),
                                                P(s["dres"].data_ptr()) if with_dres else None,
                                                P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                                P(s["dx"].data_ptr()), P(s["dw"].data_ptr()), rows, H,
                                                wsp, ws_bytes, stream))
        elif rc:
            _lib.check(lib.rmsnorm_bwd_recompute(P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv,
                                                 P(w.data_ptr()), wdt, ctypes.c_float(wl.eps), det,
                                                 P(s["dx"].data_ptr()), dxv, P(s["dw"].data_ptr()),
                                                 wsp, ws_bytes, stream))
        else:
            _lib.check(lib.rmsnorm_bwd_strided(P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv,
                                               P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                               P(s["dx"].data_ptr()), dxv, P(s["dw"].data_ptr()),
                                               wsp, ws_bytes, stream))

    def step(s, det: int, stream):
        for _ in range(n_fwd):
            fwd(s, stream)
        if has_bwd:
            bwd(s, det, stream)

    t = time_steps(args, torch, rn, _lib, dev, sets, fwd, step, n_fwd, has_bwd, ["dx", "dw"],
                   step_bytes, fwd_b, bwd_row_b, bwd_b)
    dom_name, value = t["dom_name"], t["value"]

    traffic = None
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(tr_path) and op == "fwd+bwd":
        from bwd_rmsnorm_fwd_02_amd import build as _b
        rec = json.load(open(tr_path))
        if rec.get("source_hash") == _b.source_hash() and dom_name in rec.get("kernels", {}):
            traffic = rec["kernels"][dom_name]["bytes_per_launch"]

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the same work as one step: the forward (n_fwd times; the recompute
        # backward is the forward's statistics plus the backward), then the
        # backward at the oracle's rstd
        xo = wl.x if not residual else oracle.residual_add(wl.x, wl.r)
        w64 = wl.w.f64
        r_all, _ = oracle.fwd(xo, w64, wl.eps, want_y=False)

        def oracle_rows(lo, hi):
            r64 = r_all[lo:hi]
            for _ in range(n_fwd):
                r64, _ = oracle.fwd(xo[lo:hi], w64, wl.eps)
            if rc:
                r64, _ = oracle.fwd(xo[lo:hi], w64, wl.eps, want_y=False)
            if has_bwd:
                oracle.bwd(wl.dy[lo:hi], xo[lo:hi], r64, w64)

        cpu = cpu_baseline(args, rows, step_bytes, op, oracle_rows)

    config = {"workload": args.config, "op": op, "T": T, "heads": heads, "H": H,
              "w_dtype": wl.w.dtype, "residual": residual, "deterministic": True,
              "global_batch": rows, "seq_len": T, "parallelism": "none (1 GPU)",
              "buffer_sets": n_sets}
    metric = METRIC if op == "fwd+bwd" else f"RMSNorm {op} effective HBM GB/s, per (T,H)"
    # the launch shapes, partition and load policy the route chose (host-side query)
    wt = torch.bfloat16 if wl.w.dtype == "bf16" else torch.float32
    route = {"fwd": rn.rmsnorm_route_query("fwd", rows, H, wt, residual=residual),
             "bwd": rn.rmsnorm_route_query("bwd", rows, H, wt, residual=residual,
                                           recompute=(op == "fwd+bwd_recompute"))}
    out = result_line(args, metric, op, value, t, step_bytes, config, traffic, cpu, route)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
