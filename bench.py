#!/usr/bin/env python3
"""RMSNorm-for-training throughput on one MI355X: fwd + bwd effective HBM GB/s.

A step is one pass of the whole path over one batch: the forward
(x -> y, rstd) and the deterministic backward (dy, x, rstd -> dx, dw). The
headline workload is the largest of the pages' five, x[T=131072, H=2048] BF16
with an FP32 weight and 1 % of the rows scaled by 8 (pass --config for the
others). Inputs are seeded synthetic tensors already resident in HBM.
Consecutive steps rotate over enough buffer sets (>= 1 GiB in the cycle) that
no step finds its tensors in the 256 MB Infinity Cache, so the figure is an
HBM figure.

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
  fwd+bwd_deferred     forward, then the backward that leaves its dw partial
                       rows; the K steps of a replay end with one batched
                       reduce of their K dw (a model whose layers' dw are
                       reduced together at the end of the backward). Not the
                       metric's step: reported beside it, in per_config

Timing (the pages' protocol, Cake page "Measurement", on HIP graphs):
* a replay is one HIP graph holding K = --steps steps; its GPU span is
  timed with two events on the replay stream. Each graph is replayed
  --replays times (201), split over --rounds (3) interleaved rounds in which
  the graphs take turns in a rotating order: the deterministic graph, an
  A/A second capture of the same step, and the non-deterministic graph;
* ms_per_step is the median replay span over K, with p10 and p90 beside it;
  aa_noise = |1 - median(A) / median(A')|, the noise floor of the figure;
  value = algorithmic bytes of one step / ms_per_step;
* before each round, one untimed replay of each deterministic graph is
  checked bit for bit against the eager result;
* roofline: the same steps launched eagerly (max(40, K) timed after about
  25 ms of untimed ones), each library kernel bracketed by HIP events
  recorded on its launch stream by the dispatch itself; the
  dominant kernel is the backward row kernel (the forward for --op fwd);
  achieved = its algorithmic bytes per launch / its mean duration; peak
  8 TB/s. frac_cold is the same kernel timed in backward-only steps (no
  forward before it, so nothing of x is left in the caches);
* per_config: fwd, bwd, fwd+bwd and 2xfwd+bwd (the pages' three timed ops
  and the metric's step) of every workload of the family, with the same
  protocol, in the same run (--no-per-config skips it);
* flush_protocol: cross-checks of the cold-cache setting for the chosen
  workload and op (and each workload's fwd+bwd in per_config), each a graph
  of a single step replayed --replays times: after a 512 MiB write to a
  separate buffer outside the timed span (the flush the pages run before
  each timed replay), after a 512 MiB read instead, and with no flush over
  the rotating buffer sets. Reported beside the K-step figure, never as
  value (--no-flush-check skips them);
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
FLUSH_BYTES = 512 << 20
METRIC = "RMSNorm fwd+bwd effective HBM GB/s and % of 8 TB/s peak, per (T,H)"
DEFAULT_CONFIG = "c3_T131072_H2048_f32w_heavy"
DEFAULT_LN_CONFIG = "ln_T8192_H4096_bf16w"
OPS = ("fwd+bwd", "fwd", "bwd", "2xfwd+bwd", "fwd+bwd_recompute", "fwd+bwd_deferred")
P = ctypes.c_void_p


def algorithmic_bytes(rows: int, H: int, sw: int, residual: bool, with_dres: bool):
    """Bytes the path must move per launch: (forward, backward row kernel,
    whole backward). Forward: read x (and r), write y (and h), write rstd,
    read w. Backward: read dy, x (h), (dres), rstd, w; write dx; the reduce
    writes dw."""
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


def gbps(nbytes: float, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9


def pct(v, q):
    s = sorted(v)
    if not s:
        return None
    k = (len(s) - 1) * q
    lo = math.floor(k)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


# ------------------------------------------------------------- workloads

class Work:
    """Device buffers of one workload and the library calls of its ops."""

    def __init__(self, **kw):
        self.__dict__.update(kw)

    def n_fwd(self, op):
        return {"fwd+bwd": 1, "fwd": 1, "bwd": 0, "2xfwd+bwd": 2, "fwd+bwd_recompute": 1,
                "fwd+bwd_deferred": 1}[op]

    def step_bytes(self, op):
        fwd_b, _, bwd_b = self.bytes
        if op == "fwd+bwd_recompute":
            bwd_b -= 4 * self.rows  # the recompute backward reads no rstd
        return self.n_fwd(op) * fwd_b + (bwd_b if op != "fwd" else 0)

    def step_fn(self, op):
        n_fwd, has_bwd = self.n_fwd(op), op != "fwd"
        rc = op == "fwd+bwd_recompute"

        def step(s, det, stream):
            for _ in range(n_fwd):
                self.fwd(s, stream)
            if has_bwd:
                self.bwd(s, det, stream, rc)
        return step


def n_sets_for(per_set_bytes: int) -> int:
    return int(min(16, max(2, math.ceil((1 << 30) / per_set_bytes))))


def prepare_rmsnorm(name, seed, torch, np, synth, _lib, lib, dev):
    wl = synth.config(name, seed=seed)
    rows, H, T, heads = wl.rows, wl.H, wl.T, wl.heads
    residual = wl.r is not None
    with_dres = wl.dres is not None
    sw = 2 if wl.w.dtype == "bf16" else 4
    wdt = _lib.RMSN_BF16 if sw == 2 else _lib.RMSN_F32

    def d16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    w = d16(wl.w.bits) if wl.w.dtype == "bf16" else torch.from_numpy(wl.w.f32.copy()).to(dev)
    x0 = d16(wl.xbuf if wl.xbuf is not None else wl.x)
    dy0 = d16(wl.dy)
    r0 = d16(wl.r) if residual else None
    dres0 = d16(wl.dres) if with_dres else None
    per_set = x0.numel() * 2 + dy0.numel() * 2 + 2 * rows * H * 2 * (2 if residual else 1)
    n_sets = n_sets_for(per_set)
    sets = []
    for _ in range(n_sets):
        s = dict(x=x0.clone(), dy=dy0.clone(), y=torch.empty(rows, H, dtype=torch.bfloat16, device=dev),
                 # the strided form's gap columns are never written: zero them so
                 # the replay check (which zeroes outputs first) sees the same gap
                 dx=(torch.zeros_like(x0) if wl.xbuf is not None
                     else torch.empty(rows, H, dtype=torch.bfloat16, device=dev)),
                 rstd=torch.empty(rows, dtype=torch.float32, device=dev),
                 dw=torch.empty(H, dtype=torch.float32, device=dev))
        if residual:
            s["r"] = r0.clone()
            s["h"] = torch.empty(rows, H, dtype=torch.bfloat16, device=dev)
            s["dres"] = dres0.clone() if with_dres else None
        sets.append(s)
    del x0, dy0, r0, dres0
    # one workspace per mode, so the two graphs never share one
    ws = {}
    for det in (0, 1):
        nb = max(lib.rmsnorm_bwd_workspace_bytes(rows, H, wdt, det), 256)
        raw = torch.empty(nb + 256, dtype=torch.uint8, device=dev)
        ws[det] = (raw, P(raw.data_ptr() + (-raw.data_ptr()) % 256), nb)
    if wl.xbuf is not None:
        xv = _lib.View(T, heads, H, wl.x_stride_t, wl.x_stride_h)
    else:
        xv = _lib.View(T, heads, H, heads * H, H)
    cv = _lib.View(T, heads, H, heads * H, H)
    dxv = xv if wl.xbuf is not None else cv
    eps = ctypes.c_float(wl.eps)

    def fwd(s, stream):
        if residual:
            _lib.check(lib.rmsnorm_residual_fwd(P(s["x"].data_ptr()), P(s["r"].data_ptr()),
                                                P(w.data_ptr()), wdt, eps, P(s["h"].data_ptr()),
                                                P(s["y"].data_ptr()), P(s["rstd"].data_ptr()),
                                                rows, H, stream))
        else:
            _lib.check(lib.rmsnorm_fwd_strided(P(s["x"].data_ptr()), xv, P(w.data_ptr()), wdt, eps,
                                               P(s["y"].data_ptr()), cv, P(s["rstd"].data_ptr()),
                                               stream))

    def bwd(s, det, stream, rc=False):
        _, wsp, nb = ws[det]
        if residual:
            _lib.check(lib.rmsnorm_residual_bwd(P(s["dy"].data_ptr()), P(s["h"].data_ptr()),
                                                P(s["dres"].data_ptr()) if with_dres else None,
                                                P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                                P(s["dx"].data_ptr()), P(s["dw"].data_ptr()), rows, H,
                                                wsp, nb, stream))
        elif rc:
            _lib.check(lib.rmsnorm_bwd_recompute(P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv,
                                                 P(w.data_ptr()), wdt, eps, det,
                                                 P(s["dx"].data_ptr()), dxv, P(s["dw"].data_ptr()),
                                                 wsp, nb, stream))
        else:
            _lib.check(lib.rmsnorm_bwd_strided(P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv,
                                               P(s["rstd"].data_ptr()), P(w.data_ptr()), wdt, det,
                                               P(s["dx"].data_ptr()), dxv, P(s["dw"].data_ptr()),
                                               wsp, nb, stream))

    def deferred_slots(K):
        """K partial-row buffers and dw outputs, one per step of a replay, and
        the job table of their one batched reduce."""
        need = lib.rmsnorm_bwd_partials_bytes(rows, H, wdt)
        slots = []
        for _ in range(K):
            raw = torch.empty(need + 256, dtype=torch.uint8, device=dev)
            slots.append(dict(raw=raw, ptr=raw.data_ptr() + (-raw.data_ptr()) % 256, nb=need,
                              dw=torch.empty(H, dtype=torch.float32, device=dev)))
        jobs = (_lib.DwJob * K)(*[_lib.DwJob(sl["ptr"], sl["nb"], rows, H, wdt, sl["dw"].data_ptr())
                                  for sl in slots])
        return dict(slots=slots, jobs=jobs, n=K)

    def bwd_partial(s, slot, stream):
        if residual:
            _lib.check(lib.rmsnorm_residual_bwd_strided_partials(
                P(s["dy"].data_ptr()), cv, P(s["h"].data_ptr()), cv,
                P(s["dres"].data_ptr()) if with_dres else None, cv, P(s["rstd"].data_ptr()),
                P(w.data_ptr()), wdt, P(s["dx"].data_ptr()), cv, P(slot["ptr"]), slot["nb"], stream))
        else:
            _lib.check(lib.rmsnorm_bwd_strided_partials(
                P(s["dy"].data_ptr()), cv, P(s["x"].data_ptr()), xv, P(s["rstd"].data_ptr()),
                P(w.data_ptr()), wdt, P(s["dx"].data_ptr()), dxv, P(slot["ptr"]), slot["nb"], stream))

    def reduce_slots(d, stream):
        _lib.check(lib.rmsnorm_dw_reduce_batch(d["jobs"], d["n"], stream))

    return Work(name=name, norm="rmsnorm", wl=wl, rows=rows, T=T, heads=heads, H=H,
                residual=residual, with_dres=with_dres, wdtype=wl.w.dtype, sets=sets, ws=ws,
                fwd=fwd, bwd=bwd, out_keys=("y", "dx", "dw"), deferred_slots=deferred_slots,
                bwd_partial=bwd_partial, reduce_slots=reduce_slots,
                bytes=algorithmic_bytes(rows, H, sw, residual, with_dres))


def prepare_layernorm(name, seed, torch, np, synth, _lib, lib, dev):
    wl = synth.ln_config(name, seed=seed)
    T, H = wl.T, wl.H
    sw = 2 if wl.gamma.dtype == "bf16" else 4
    wdt = _lib.RMSN_BF16 if sw == 2 else _lib.RMSN_F32

    def d16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def wdev(wt):
        return d16(wt.bits) if wt.dtype == "bf16" else torch.from_numpy(wt.f32.copy()).to(dev)

    gam, bet = wdev(wl.gamma), wdev(wl.beta)
    x0, dy0 = d16(wl.x), d16(wl.dy)
    n_sets = n_sets_for(4 * T * H * 2)
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

    def bwd(s, det, stream, rc=False):
        _, wsp, nb = ws[det]
        _lib.check(lib.layernorm_bwd(P(s["dy"].data_ptr()), P(s["x"].data_ptr()),
                                     P(s["mean"].data_ptr()), P(s["rstd"].data_ptr()),
                                     P(gam.data_ptr()), wdt, det, P(s["dx"].data_ptr()),
                                     P(s["dg"].data_ptr()), P(s["db"].data_ptr()), T, H, wsp, nb,
                                     stream))

    return Work(name=name, norm="layernorm", wl=wl, rows=T, T=T, heads=1, H=H, residual=False,
                with_dres=False, wdtype=wl.gamma.dtype, sets=sets, ws=ws, fwd=fwd, bwd=bwd,
                out_keys=("y", "dx", "dg", "db"), bytes=ln_algorithmic_bytes(T, H, sw))


# --------------------------------------------------------------- timing

def same_bits(torch, a, b):
    va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
    vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
    return torch.equal(va, vb)


def measure_op(args, torch, rn, _lib, dev, wk, op, nondet=True):
    """Graph-replay timing of K steps of `op` under the replay protocol, and
    per-kernel event timing of the same K steps launched eagerly."""
    sets = wk.sets
    n_sets = len(sets)
    K, W = args.steps, args.warmup
    cur = torch.cuda.current_stream(dev)
    sp = P(cur.cuda_stream)
    deferred = op == "fwd+bwd_deferred"
    step = None if deferred else wk.step_fn(op)
    dslots = wk.deferred_slots(K) if deferred else None
    has_bwd = op != "fwd"
    out_keys = [k for k in wk.out_keys if (k == "y" and wk.n_fwd(op)) or (k != "y" and has_bwd)]

    def run(i0, n, det, stream):
        """Steps i0 .. i0 + n - 1. Deferred: n is a multiple of K, and each K
        steps (forward, backward leaving its partial rows in slot k) end with
        the one batched reduce of their K dw."""
        if not deferred:
            for i in range(i0, i0 + n):
                step(sets[i % n_sets], det, stream)
            return
        for g0 in range(i0, i0 + n, K):
            for k in range(K):
                s = sets[(g0 + k) % n_sets]
                wk.fwd(s, stream)
                wk.bwd_partial(s, dslots["slots"][k], stream)
            wk.reduce_slots(dslots, stream)

    def outputs():
        o = {k: sets[0][k] for k in out_keys}
        if deferred:
            o["dw"] = dslots["slots"][0]["dw"]
        return o

    # every set gets a forward's rstd (and h) first, so a backward-only step
    # has its inputs; then the eager warm-up and a reference result for set 0
    for s in sets:
        wk.fwd(s, sp)
    if deferred:
        for _ in range(max(1, math.ceil(W / K))):
            run(0, K, 1, sp)
    else:
        run(0, max(1, W), 1, sp)  # at least one step: set 0's outputs are the reference
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outputs().items()}

    def capture(det: int):
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream(device=dev)
        cs.wait_stream(cur)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                csp = P(torch.cuda.current_stream(dev).cuda_stream)
                run(0, K, det, csp)
        torch.cuda.synchronize()
        return g

    graphs = [("det", capture(1)), ("det_aa", capture(1))]
    if nondet and has_bwd and not deferred:
        graphs.append(("nondet", capture(0)))

    def check(g, tag):
        for t in outputs().values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outputs().items():
            assert same_bits(torch, t, ref[k]), f"{wk.name} {op} {tag}: graph {k} != eager"

    rounds = max(1, args.rounds)
    per_round = max(1, math.ceil(args.replays / rounds))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(per_round)]
    spans = {k: [] for k, _ in graphs}
    for rnd in range(rounds):
        order = graphs[rnd % len(graphs):] + graphs[:rnd % len(graphs)]
        for key, g in order:
            if key != "nondet":
                check(g, key)
            else:
                g.replay()  # untimed, as the deterministic graphs' checked replay
            for i in range(per_round):
                ev[i][0].record(cur)
                g.replay()
                ev[i][1].record(cur)
            torch.cuda.synchronize()
            spans[key] += [ev[i][0].elapsed_time(ev[i][1]) for i in range(per_round)]
    del graphs

    def stats(v):
        return {"median": pct(v, 0.5) / K, "p10": pct(v, 0.1) / K, "p90": pct(v, 0.9) / K,
                "replays": len(v)}

    st = {k: stats(v) for k, v in spans.items()}
    aa = abs(1.0 - st["det"]["median"] / st["det_aa"]["median"])

    # Per-kernel HIP-event timing of the same steps, launched eagerly. The
    # GPU is first parked on a sleep kernel so that the host queues the steps
    # before they run: the kernels then run back to back and each event pair
    # brackets GPU time only, not host launch gaps. The first k_warm queued
    # steps, about 25 ms of GPU work, are not timed: the kernels right after
    # the idle sleep run slower while the part ramps back up (at 8192 x 8192
    # LayerNorm, 2.5 ms of warm-up left its backward 25 % slower than 25 ms).
    step_ms = st["det"]["median"]
    k_warm = int(min(1000, max(10, K, math.ceil(25.0 / max(step_ms, 1e-3)))))
    k_timed = max(40, K)
    if deferred:  # whole groups of K steps
        k_warm, k_timed = K * math.ceil(k_warm / K), K * math.ceil(k_timed / K)
    rn.rmsnorm_timing_read()
    rn.rmsnorm_timing_enable(False)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    t0 = time.perf_counter()
    run(0, k_warm, 1, sp)
    rn.rmsnorm_timing_enable(True)
    run(k_warm, k_timed, 1, sp)
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    timers = rn.rmsnorm_timing_read()
    rn.rmsnorm_timing_enable(False)

    def avg_us(idx):
        n, ms = timers[idx]
        return (ms / n * 1e3) if n else None

    ku = {"fwd": avg_us(_lib.RMSN_TIMER_FWD), "bwd_row": avg_us(_lib.RMSN_TIMER_BWD_ROW),
          "dw_reduce": avg_us(_lib.RMSN_TIMER_DW_REDUCE), "bwd_small": avg_us(_lib.RMSN_TIMER_BWD_SMALL)}
    sb = wk.step_bytes(op)
    ms = st["det"]["median"]
    return {"op": op, "step_bytes": sb, "ms_per_step": ms, "stats": st, "aa_noise": aa,
            "value": gbps(sb, ms), "kernel_us": ku, "t_issue_ms": t_issue * 1e3 / (k_warm + k_timed),
            "K": K, "W": W, "kernel_steps": k_timed}


def measure_flush(args, torch, dev, wk, op):
    """Cross-checks of the cold-cache setting, each --replays replays of a
    graph holding a single step, timed with HIP events around the replay:
      write_flush: 512 MiB written to a separate buffer before each replay,
        outside the span (the flush the pages run before each timed replay);
        the step starts with the caches full of that buffer's dirty lines;
      read_flush: the same buffer read (summed) instead, which evicts the
        step's tensors without leaving dirty lines behind;
      one_step_rotating: no flush; one single-step graph per buffer set,
        replayed in rotation, so the step is as cold as in the K-step graphs
        and only the per-replay launch cost differs from them.
    Run after measure_op on the same workload, so every buffer set already
    holds a forward's outputs."""
    cur = torch.cuda.current_stream(dev)
    step = wk.step_fn(op)
    graphs = []
    for s in wk.sets:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream(device=dev)
        cs.wait_stream(cur)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                step(s, 1, P(torch.cuda.current_stream(dev).cuda_stream))
        graphs.append(g)
    torch.cuda.synchronize()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    n = max(1, args.replays)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    sb = wk.step_bytes(op)

    def run(prep, rotate):
        graphs[0].replay()  # untimed
        for i in range(n):
            g = graphs[i % len(graphs)] if rotate else graphs[0]
            prep(i)
            ev[i][0].record(cur)
            g.replay()
            ev[i][1].record(cur)
        torch.cuda.synchronize()
        spans = [ev[i][0].elapsed_time(ev[i][1]) for i in range(n)]
        med = pct(spans, 0.5)
        return {"ms_per_step": round(med, 5), "p10": round(pct(spans, 0.1), 5),
                "p90": round(pct(spans, 0.9), 5), "value": round(gbps(sb, med), 2)}

    sink = []

    def read_flush(i):
        sink.append(flush.sum())  # results kept briefly, so the reads are not elided
        if len(sink) > 64:
            sink.clear()

    out = {"replays": n, "flush_bytes": FLUSH_BYTES, "buffer_sets": len(graphs),
           "span": "HIP events around one replay of a one-step graph"}
    out["write_flush"] = run(lambda i: flush.fill_(float(i & 1023)), False)
    out["read_flush"] = run(read_flush, False)
    out["one_step_rotating"] = run(lambda i: None, True)
    del graphs, flush, sink
    torch.cuda.empty_cache()
    return out


def dominant(wk, op, m):
    """The dominant kernel of a step: (name, algorithmic bytes, mean us)."""
    fwd_b, bwd_row_b, bwd_b = wk.bytes
    ku = m["kernel_us"]
    if op == "fwd+bwd_recompute":
        bwd_row_b -= 4 * wk.rows
        bwd_b -= 4 * wk.rows
    if op == "fwd":
        return "fwd", fwd_b, ku["fwd"]
    if ku["bwd_row"] is not None:
        return "bwd_row", bwd_row_b, ku["bwd_row"]
    return "bwd_small", bwd_b, ku["bwd_small"]


def op_summary(wk, op, m):
    st = m["stats"]["det"]
    name, nb, us = dominant(wk, op, m)
    traffic = traffic_for(wk.name, name) if op == "fwd+bwd" else None  # counted in fwd+bwd steps
    out = {"GBps": round(m["value"], 1), "pct_of_hbm_peak": round(100 * m["value"] / HBM_PEAK_GBPS, 2),
           "ms_per_step": round(m["ms_per_step"], 5), "p10": round(st["p10"], 5),
           "p90": round(st["p90"], 5), "aa_noise": round(m["aa_noise"], 4),
           "kernel_us": {k: (round(v, 3) if v is not None else None) for k, v in m["kernel_us"].items()},
           "roofline_kernel": name,
           "roofline_frac": round(gbps(nb, us * 1e-3) / HBM_PEAK_GBPS, 4) if us else None,
           "roofline_bytes": nb, "traffic": traffic}
    if "nondet" in m["stats"]:
        out["nondet_ms_per_step"] = round(m["stats"]["nondet"]["median"], 5)
    return out


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


def oracle_step(wk, op):
    """The oracle's work of one step on rows [lo, hi) (test infrastructure,
    imported only for the CPU baseline)."""
    import oracle
    wl = wk.wl
    n_fwd, has_bwd, rc = wk.n_fwd(op), op != "fwd", op == "fwd+bwd_recompute"
    if wk.norm == "layernorm":
        g64, b64 = wl.gamma.f64, wl.beta.f64
        mu_all, rs_all, _ = oracle.ln_fwd(wl.x, g64, b64, wl.eps, want_y=False)

        def rows_fn(lo, hi):
            mu, rs = mu_all[lo:hi], rs_all[lo:hi]
            for _ in range(n_fwd):
                mu, rs, _ = oracle.ln_fwd(wl.x[lo:hi], g64, b64, wl.eps)
            if has_bwd:
                oracle.ln_bwd(wl.dy[lo:hi], wl.x[lo:hi], mu, rs, g64)
        return rows_fn
    xo = wl.x if wl.r is None else oracle.residual_add(wl.x, wl.r)
    w64 = wl.w.f64
    r_all, _ = oracle.fwd(xo, w64, wl.eps, want_y=False)

    def rows_fn(lo, hi):
        r64 = r_all[lo:hi]
        for _ in range(n_fwd):
            r64, _ = oracle.fwd(xo[lo:hi], w64, wl.eps)
        if rc:
            r64, _ = oracle.fwd(xo[lo:hi], w64, wl.eps, want_y=False)
        if has_bwd:
            oracle.bwd(wl.dy[lo:hi], xo[lo:hi], r64, w64)
    return rows_fn


def traffic_for(config, dom_name):
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(tr_path):
        return None
    from bwd_rmsnorm_fwd_02_amd import build as _b
    rec = json.load(open(tr_path))
    if rec.get("source_hash") == _b.source_hash() and dom_name in rec.get("kernels", {}):
        return rec["kernels"][dom_name]["bytes_per_launch"]
    return None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per graph replay (K)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--norm", choices=("rmsnorm", "layernorm"), default="rmsnorm")
    ap.add_argument("--config", default=None)
    ap.add_argument("--op", choices=OPS, default="fwd+bwd")
    ap.add_argument("--replays", type=int, default=201, help="replays per graph")
    ap.add_argument("--rounds", type=int, default=3, help="interleaved rounds the replays are split over")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the chosen workload, not every workload of its family")
    ap.add_argument("--no-flush-check", action="store_true",
                    help="skip the flush-protocol cross-check of the chosen workload and op")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the backward-only (cold) timing of the chosen workload, so that "
                         "a kernel trace holds the in-step launches of its kernels only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of oracle work for each of the two CPU runs")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle run (0: min(16, CPUs))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 10 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.replays < 1 or args.rounds < 1:
        print("--steps, --replays and --rounds take 1 or more, --warmup 0 or more", file=sys.stderr)
        return 2

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

    ln = args.norm == "layernorm"
    if ln and args.op not in ("fwd+bwd", "fwd", "bwd", "2xfwd+bwd"):
        print("--norm layernorm takes --op fwd+bwd, fwd, bwd or 2xfwd+bwd", file=sys.stderr)
        return 2
    if args.config is None:
        args.config = DEFAULT_LN_CONFIG if ln else DEFAULT_CONFIG
    prepare = prepare_layernorm if ln else prepare_rmsnorm
    family = list(synth.LN_CONFIGS) if ln else list(synth.CONFIGS)

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------- the chosen workload and op
    progress(f"{args.config}: generating inputs")
    wk = prepare(args.config, args.seed, torch, np, synth, _lib, lib, dev)
    op = args.op
    if op == "fwd+bwd_recompute" and wk.residual:
        print("--op fwd+bwd_recompute covers the plain and per-head forms only", file=sys.stderr)
        return 2
    progress(f"{args.config} {op}: timing")
    m = measure_op(args, torch, rn, _lib, dev, wk, op)
    cold = None
    if op != "fwd" and op != "bwd" and not args.no_cold:
        progress(f"{args.config} bwd alone: timing (cold backward)")
        cold = measure_op(args, torch, rn, _lib, dev, wk, "bwd", nondet=False)
    flush_m = None
    if not args.no_flush_check and op != "fwd+bwd_deferred":
        progress(f"{args.config} {op}: flush-protocol cross-check")
        flush_m = measure_flush(args, torch, dev, wk, op)
    dom_name, dom_bytes, dom_us = dominant(wk, op, m)
    achieved = gbps(dom_bytes, dom_us * 1e-3)
    frac_cold = None
    if cold is not None and dom_name == "bwd_row" and cold["kernel_us"]["bwd_row"]:
        frac_cold = gbps(dom_bytes, cold["kernel_us"]["bwd_row"] * 1e-3) / HBM_PEAK_GBPS
    cpu = None
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle)")
        cpu = cpu_baseline(args, wk.rows, wk.step_bytes(op), op, oracle_step(wk, op))
    wt = torch.bfloat16 if wk.wdtype == "bf16" else torch.float32
    if ln:
        route = {"fwd": rn.rmsnorm_route_query("ln_fwd", wk.rows, wk.H, wt),
                 "bwd": rn.rmsnorm_route_query("ln_bwd", wk.rows, wk.H, wt)}
    else:
        route = {"fwd": rn.rmsnorm_route_query("fwd", wk.rows, wk.H, wt, residual=wk.residual),
                 "bwd": rn.rmsnorm_route_query("bwd", wk.rows, wk.H, wt, residual=wk.residual,
                                               recompute=(op == "fwd+bwd_recompute"))}
    head_rows, head_T, head_heads, head_H = wk.rows, wk.T, wk.heads, wk.H
    head_res, head_wdt, n_sets = wk.residual, wk.wdtype, len(wk.sets)
    per_config = {}
    if op == "fwd+bwd":
        per_config[args.config] = {"fwd+bwd": op_summary(wk, op, m)}
        if flush_m is not None:
            per_config[args.config]["fwd+bwd"]["flush_protocol"] = flush_m
        if cold is not None:
            per_config[args.config]["bwd"] = op_summary(wk, "bwd", cold)
    del wk
    torch.cuda.empty_cache()

    # ---------------- every workload of the family: fwd, bwd, fwd+bwd
    if not args.no_per_config:
        for name in family:
            progress(f"per-config {name}: generating inputs")
            w2 = prepare(name, args.seed, torch, np, synth, _lib, lib, dev)
            entry = per_config.setdefault(name, {})
            ops = ("fwd+bwd", "bwd", "fwd", "2xfwd+bwd") + (() if ln else ("fwd+bwd_deferred",))
            for o in ops:
                if o in entry:
                    continue
                progress(f"per-config {name} {o}: timing")
                entry[o] = op_summary(w2, o, measure_op(args, torch, rn, _lib, dev, w2, o))
            if not args.no_flush_check and "flush_protocol" not in entry["fwd+bwd"]:
                progress(f"per-config {name} fwd+bwd: flush-protocol cross-check")
                entry["fwd+bwd"]["flush_protocol"] = measure_flush(args, torch, dev, w2, "fwd+bwd")
            if "bwd" in entry and entry["bwd"]["roofline_kernel"] == "bwd_row":
                entry["fwd+bwd"]["roofline_frac_cold_bwd"] = entry["bwd"]["roofline_frac"]
            wt2 = torch.bfloat16 if w2.wdtype == "bf16" else torch.float32
            if ln:
                entry["route"] = {"fwd": rn.rmsnorm_route_query("ln_fwd", w2.rows, w2.H, wt2),
                                  "bwd": rn.rmsnorm_route_query("ln_bwd", w2.rows, w2.H, wt2)}
            else:
                entry["route"] = {"fwd": rn.rmsnorm_route_query("fwd", w2.rows, w2.H, wt2,
                                                                residual=w2.residual),
                                  "bwd": rn.rmsnorm_route_query("bwd", w2.rows, w2.H, wt2,
                                                                residual=w2.residual)}
            del w2
            torch.cuda.empty_cache()

    K = m["K"]
    st = m["stats"]
    value = m["value"]
    metric = (METRIC if op == "fwd+bwd" else f"RMSNorm {op} effective HBM GB/s, per (T,H)")
    if ln:
        metric = f"LayerNorm {op} effective HBM GB/s, per (T,H)"
    config = {"workload": args.config, "norm": args.norm, "op": op, "T": head_T, "heads": head_heads,
              "H": head_H, "w_dtype": head_wdt, "residual": head_res, "deterministic": True,
              "global_batch": head_rows, "seq_len": head_T, "parallelism": "none (1 GPU)",
              "buffer_sets": n_sets, "steps_per_replay": K}
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": m["W"],
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic: FP32 row math with FP64 sums (rstd, dw); BF16 and the
        # weight dtype are storage only
        "dtype": "f32",
        "io_dtype": "bf16 activations and gradients, weight as configured",
        "data": "synthetic",
        "config": config,
        "p10": round(st["det"]["p10"], 5),
        "p90": round(st["det"]["p90"], 5),
        "aa_noise": round(m["aa_noise"], 4),
        "timing": {"replays": st["det"]["replays"], "rounds": args.rounds, "steps_per_replay": K,
                   "span": "HIP events around each graph replay on the replay stream",
                   "ms_per_step": {k: {q: round(v, 5) for q, v in s.items() if q != "replays"}
                                   for k, s in st.items()},
                   "value_p90_p10_GBps": [round(gbps(m["step_bytes"], st["det"]["p90"]), 1),
                                          round(gbps(m["step_bytes"], st["det"]["p10"]), 1)]},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "nondeterministic": ({"ms_per_step": round(st["nondet"]["median"], 5),
                              "value": round(gbps(m["step_bytes"], st["nondet"]["median"]), 2),
                              "route": "the same fixed-order kernels as the deterministic mode"}
                             if "nondet" in st else None),
        "kernel_us": m["kernel_us"],
        "eager_host_issue_ms_per_step": round(m["t_issue_ms"], 5),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(args.config, dom_name) if op == "fwd+bwd" else None,
                     "algorithmic_bytes": dom_bytes,
                     "frac_cold": round(frac_cold, 4) if frac_cold is not None else None},
        "flush_protocol": flush_m,
        "cpu_baseline": cpu,
        "route": route,
        "per_config": per_config or None,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
