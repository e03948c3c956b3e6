#!/usr/bin/env python3
"""RMSNorm-for-training throughput on one MI355X: fwd + bwd effective HBM GB/s.

A step is one pass of the whole path over one batch: the forward
(x -> y, rstd) and the deterministic backward (dy, x, rstd -> dx, dw) of the
RMSNorm workload x[T=4096, H=4096] BF16 with a BF16 weight (the workload the
metric is quoted on; pass --config for the others). Inputs are seeded
synthetic tensors already resident in HBM. Consecutive steps rotate over
enough buffer sets (>= 1 GiB in the cycle) that no step finds its tensors in
the 256 MB Infinity Cache, so the figure is an HBM figure.

Timing:
* value: K steps captured in one HIP graph (the pages time graph replays),
  replayed once between two synchronisations; GB/s of algorithmic bytes.
* roofline: the same K steps launched eagerly with the library's per-kernel
  HIP-event timers on the launch stream; the dominant kernel is the
  backward row kernel; achieved = its algorithmic bytes per launch / its
  mean event-timed duration; peak = 8 TB/s.
* cpu_baseline: the FP64 oracle, single-threaded, on the same workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
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


def algorithmic_bytes(rows: int, H: int, sw: int, residual: bool, with_dres: bool):
    """Bytes the path must move (per launch): see the design doc, measurement."""
    e = rows * H
    fwd = (8 if residual else 4) * e + 4 * rows + H * sw
    bwd_row = ((8 if with_dres else 6) if residual else 6) * e + 4 * rows + H * sw
    bwd = bwd_row + 4 * H
    return fwd, bwd_row, bwd


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
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

    wl = synth.config(args.config, seed=args.seed)
    rows, H, T, heads = wl.rows, wl.H, wl.T, wl.heads
    residual = wl.r is not None
    with_dres = wl.dres is not None
    sw = 2 if wl.w.dtype == "bf16" else 4
    wdt = _lib.RMSN_BF16 if wl.w.dtype == "bf16" else _lib.RMSN_F32
    fwd_b, bwd_row_b, bwd_b = algorithmic_bytes(rows, H, sw, residual, with_dres)
    step_bytes = fwd_b + bwd_b

    def d16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

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
                 dx=torch.empty_like(x0) if wl.xbuf is not None else torch.empty(rows, H, dtype=torch.bfloat16, device=dev),
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
    P = ctypes.c_void_p
    ws_arg = {1: (P(ws_det.data_ptr()), ws_bytes_det), 0: (P(ws_nd.data_ptr()), ws_bytes_nd)}

    if wl.xbuf is not None:
        xv = _lib.View(T, heads, H, wl.x_stride_t, wl.x_stride_h)
    else:
        xv = _lib.View(T, heads, H, heads * H, H)
    cv = _lib.View(T, heads, H, heads * H, H)

    def step(s, det: int, stream):
        wsp, ws_bytes = ws_arg[det]
        if residual:
            _lib.check(lib.rmsnorm_residual_fwd(P(s["x"].data_ptr()), P(s["r"].data_ptr()),
                                                P(w.data_ptr()), wdt, ctypes.c_float(wl.eps),
                                                P(s["h"].data_ptr()), P(s["y"].data_ptr()),
                                                P(s["rstd"].data_ptr()), rows, H, stream))
            _lib.check(lib.rmsnorm_residual_bwd(P(s["dy"].data_ptr()), P(s["h"].data_ptr()),
                                                P(s["dres"].data_ptr()) if with_dres else None,
                                                P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                                P(s["dx"].data_ptr()), P(s["dw"].data_ptr()), rows, H,
                                                wsp, ws_bytes, stream))
        else:
            _lib.check(lib.rmsnorm_fwd_strided(P(s["x"].data_ptr()), xv, P(w.data_ptr()), wdt,
                                               ctypes.c_float(wl.eps), P(s["y"].data_ptr()), cv,
                                               P(s["rstd"].data_ptr()), stream))
            _lib.check(lib.rmsnorm_bwd_strided(P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv,
                                               P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                               P(s["dx"].data_ptr()), xv if wl.xbuf is not None else cv,
                                               P(s["dw"].data_ptr()), wsp, ws_bytes, stream))

    K, W = args.steps, args.warmup
    cur = torch.cuda.current_stream(dev)
    sp = P(cur.cuda_stream)

    # eager warm-up, then a reference result for set 0
    for i in range(W):
        step(sets[i % n_sets], 1, sp)
    torch.cuda.synchronize()
    ref_dx = sets[0]["dx"].clone()
    ref_dw = sets[0]["dw"].clone()

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

    def timed_replay(g):
        g.replay()  # warm
        torch.cuda.synchronize()
        sets[0]["dx"].zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3, e0.elapsed_time(e1)

    g_det = capture(1)
    wall_ms, gpu_ms = timed_replay(g_det)
    # every replay must reproduce the eager deterministic result
    assert torch.equal(sets[0]["dx"].view(torch.int16), ref_dx.view(torch.int16)), "graph dx != eager"
    assert torch.equal(sets[0]["dw"].view(torch.int32), ref_dw.view(torch.int32)), "graph dw != eager"
    del g_det
    g_nd = capture(0)
    wall_nd_ms, gpu_nd_ms = timed_replay(g_nd)
    del g_nd

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
    if bwd_row_us is not None:
        dom_name, dom_us, dom_bytes = "bwd_row", bwd_row_us, bwd_row_b
    else:
        dom_name, dom_us, dom_bytes = "bwd_small", small_us, bwd_b
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    traffic = None
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{args.config}.json")
    if os.path.exists(tr_path):
        from bwd_rmsnorm_fwd_02_amd import build as _b
        rec = json.load(open(tr_path))
        if rec.get("source_hash") == _b.source_hash() and dom_name in rec.get("kernels", {}):
            traffic = rec["kernels"][dom_name]["bytes_per_launch"]

    fwd_gbps = fwd_b / (fwd_us * 1e-6) / 1e9 if fwd_us else None
    bwd_us = (bwd_row_us or 0.0) + (reduce_us or 0.0) if bwd_row_us else small_us
    bwd_gbps = bwd_b / (bwd_us * 1e-6) / 1e9 if bwd_us else None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t_start = time.perf_counter()
        reps = 0
        # the whole workload: forward, then backward at the oracle's rstd
        xo = wl.x if not residual else oracle.residual_add(wl.x, wl.r)
        while True:
            r64, y64 = oracle.fwd(xo, wl.w.f64, wl.eps)
            oracle.bwd(wl.dy, xo, r64, wl.w.f64)
            reps += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds:
                break
        cpu_gbps = step_bytes * reps / el / 1e9
        model = ""
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(cpu_gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the full {args.config} workload (fwd + bwd, FP64), {reps} repetition(s) "
                         f"in {el:.1f} s on one thread of {model or platform.processor()}"}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.config, "T": T, "heads": heads, "H": H,
                   "w_dtype": wl.w.dtype, "residual": residual, "deterministic": True,
                   "global_batch": rows, "seq_len": T, "parallelism": "none (1 GPU)",
                   "buffer_sets": n_sets},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "fwd_GBps": round(fwd_gbps, 1) if fwd_gbps else None,
        "bwd_GBps": round(bwd_gbps, 1) if bwd_gbps else None,
        "nondeterministic": {"ms_per_step": round(wall_nd_ms / K, 5),
                             "value": round(step_bytes / (wall_nd_ms / K * 1e-3) / 1e9, 2)},
        "kernel_us": {"fwd": fwd_us, "bwd_row": bwd_row_us, "dw_reduce": reduce_us,
                      "bwd_small": small_us},
        "graph_gpu_ms": round(gpu_ms, 4),
        "eager_host_issue_ms_per_step": round(t_issue * 1e3 / K, 5),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": dom_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
