"""The deferred dw reduction: rmsnorm_bwd_strided_partials and
rmsnorm_residual_bwd_strided_partials leave the partial rows, and
rmsnorm_dw_reduce_batch reduces many of them in one launch.

Every job's dw must have exactly the bits of the deterministic
rmsnorm_bwd_strided (rmsnorm_residual_bwd_strided) call on the same inputs,
and dx (dh) the same bits too: the split runs the same kernels in the same
order. Checked over one batch mixing the plain and residual forms, views,
token counts at and below the column-task limit, zero rows, and both partial
precisions; over a batch larger than one launch's job table; and in a
captured HIP graph of several layers' backward plus one batched reduce,
replayed with eager work in between. dw is also held to the oracle's budget.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import synth
from tests.parity import check_dw, oracle_rstd32
from tests.test_parity_gpu import DEV, _announce, dev_bf16, dev_f32, dev_w, host_bits

pytestmark = pytest.mark.gpu

# (T, heads, H, weight dtype, form, gap): form "plain" or "residual"
CASES = [
    (4096, 1, 4096, "bf16", "plain", 0),      # FP32 partial rows
    (9000, 1, 2048, "f32", "plain", 0),       # FP64 partial rows
    (3001, 4, 256, "f32", "plain", 64),       # per-head view in a wider buffer
    (64, 1, 256, "f32", "plain", 0),          # column-task route: one FP32 row
    (1, 1, 1032, "bf16", "plain", 0),
    (0, 1, 512, "bf16", "plain", 0),          # zero rows: dw = 0
    (2000, 1, 6144, "bf16", "residual", 0),
    (300, 24, 256, "f32", "residual", 8),
    (33, 1, 4096, "bf16", "residual", 0),
]


def _inputs(T, heads, H, wdt, form, gap, seed):
    residual = form == "residual"
    wl = synth.make(T=max(T, 1), H=H, w_dtype=wdt, seed=seed, heads=heads, residual=residual,
                    with_dres=residual)
    rows = T * heads
    W = heads * H + gap

    def view(bits):
        buf = torch.zeros((T, W), dtype=torch.bfloat16, device=DEV)
        v = buf[:, : heads * H].unflatten(1, (heads, H))
        if rows:
            v.copy_(dev_bf16(bits[:rows]).view(T, heads, H))
        return v

    src = oracle.residual_add(wl.x, wl.r) if residual else wl.x
    _, r32 = oracle_rstd32(src[: max(rows, 1)], wl.w.f64, wl.eps)
    t = dict(x=view(src), dy=view(wl.dy), w=dev_w(wl.w), rs=dev_f32(r32[:rows]).view(T, heads),
             dres=view(wl.dres) if residual else None, rows=rows, H=H, wdt=wdt, form=form,
             src=src[:rows], dy_bits=wl.dy[:rows], w64=wl.w.f64, r32=r32[:rows])
    return t


def _reference(t):
    dx = torch.empty(t["x"].shape, dtype=torch.bfloat16, device=DEV)
    if t["form"] == "residual":
        _, dw = rn.rmsnorm_residual_bwd_strided(t["dy"], t["x"], t["rs"], t["w"], dres=t["dres"],
                                                deterministic=True, dh=dx)
    else:
        _, dw = rn.rmsnorm_bwd_strided(t["dy"], t["x"], t["rs"], t["w"], deterministic=True, dx=dx)
    return dx, dw


def _deferred(t, dx=None, partials=None):
    if t["form"] == "residual":
        return rn.rmsnorm_residual_bwd_strided_partials(t["dy"], t["x"], t["rs"], t["w"],
                                                        dres=t["dres"], dh=dx, partials=partials)
    return rn.rmsnorm_bwd_strided_partials(t["dy"], t["x"], t["rs"], t["w"], dx=dx,
                                           partials=partials)


def _job(t, partials, dw):
    wt = torch.bfloat16 if t["wdt"] == "bf16" else torch.float32
    return (partials, t["rows"], t["H"], wt, dw)


def test_deferred_batch_matches_the_backward():
    tens = [_inputs(*c, seed=300 + i) for i, c in enumerate(CASES)]
    refs = [_reference(t) for t in tens]
    outs = [_deferred(t) for t in tens]
    dws = [torch.full((t["H"],), float("nan"), dtype=torch.float32, device=DEV) for t in tens]
    rn.rmsnorm_dw_reduce_batch([_job(t, p, dw) for t, (_, p), dw in zip(tens, outs, dws)])
    torch.cuda.synchronize()
    for c, t, (dx_r, dw_r), (dx_d, _), dw in zip(CASES, tens, refs, outs, dws):
        _announce(f"deferred {c}")
        assert torch.equal(dx_d.view(torch.int16), dx_r.view(torch.int16)), f"{c}: dx differs"
        assert torch.equal(dw.view(torch.int32), dw_r.view(torch.int32)), f"{c}: dw differs"
        if t["rows"]:
            _, _, dw64 = oracle.bwd(t["dy_bits"], t["src"], t["r32"].astype(np.float64), t["w64"],
                                    want_dx=False)
            check_dw(f"dw {c}", dw.cpu().numpy(), dw64)
        else:
            assert not torch.any(dw), f"{c}: dw over zero rows is not zero"


def test_deferred_batch_above_one_launch():
    """40 jobs of each partial precision: more than one launch's job table."""
    tens = []
    for i in range(40):
        tens.append(_inputs(100 + 7 * i, 1, 8 * (1 + i % 5), "f32", "plain", 0, seed=500 + i))
        tens.append(_inputs(8200 + i, 1, 16 * (1 + i % 3), "bf16", "plain", 0, seed=600 + i))
    refs = [_reference(t) for t in tens]
    outs = [_deferred(t) for t in tens]
    dws = [torch.full((t["H"],), float("nan"), dtype=torch.float32, device=DEV) for t in tens]
    rn.rmsnorm_dw_reduce_batch([_job(t, p, dw) for t, (_, p), dw in zip(tens, outs, dws)])
    torch.cuda.synchronize()
    for i, ((_, dw_r), dw) in enumerate(zip(refs, dws)):
        assert torch.equal(dw.view(torch.int32), dw_r.view(torch.int32)), f"job {i}: dw differs"


def test_deferred_layers_in_a_captured_graph():
    """Three layers' backward leaving partials, then one batched reduce, in
    one HIP graph; every replay gives the eager bits."""
    tens = [_inputs(4096, 1, 4096, "bf16", "plain", 0, seed=701),
            _inputs(2048, 4, 256, "f32", "residual", 0, seed=702),
            _inputs(9000, 1, 1024, "bf16", "plain", 0, seed=703)]
    dxs = [torch.empty(t["x"].shape, dtype=torch.bfloat16, device=DEV) for t in tens]
    parts = []
    for t in tens:
        wt = torch.bfloat16 if t["wdt"] == "bf16" else torch.float32
        raw = torch.empty(rn.rmsnorm_bwd_partials_bytes(t["rows"], t["H"], wt) + 256,
                          dtype=torch.uint8, device=DEV)
        parts.append(raw[(-raw.data_ptr()) % 256:])
    dws = [torch.empty((t["H"],), dtype=torch.float32, device=DEV) for t in tens]
    jobs = [_job(t, p, dw) for t, p, dw in zip(tens, parts, dws)]

    def step():
        for t, dx, p in zip(tens, dxs, parts):
            _deferred(t, dx=dx, partials=p)
        rn.rmsnorm_dw_reduce_batch(jobs)

    step()
    torch.cuda.synchronize()
    ref = [(dx.clone(), dw.clone()) for dx, dw in zip(dxs, dws)]
    for t, (dx_r, dw_r) in zip(tens, ref):
        dx_s, dw_s = _reference(t)
        torch.cuda.synchronize()
        assert torch.equal(dx_s.view(torch.int16), dx_r.view(torch.int16))
        assert torch.equal(dw_s.view(torch.int32), dw_r.view(torch.int32))
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(device=DEV)
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.synchronize()
    for i in range(3):
        for dx, dw in zip(dxs, dws):
            dx.zero_()
            dw.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ((dx_r, dw_r), dx, dw) in enumerate(zip(ref, dxs, dws)):
            assert torch.equal(dx.view(torch.int16), dx_r.view(torch.int16)), f"replay {i} layer {k}: dx"
            assert torch.equal(dw.view(torch.int32), dw_r.view(torch.int32)), f"replay {i} layer {k}: dw"
        step()  # eager work between replays
        torch.cuda.synchronize()
