"""Seeded random shapes through the public RMSNorm and LayerNorm entry
points, against the FP64 oracle.

The hand-picked shapes elsewhere pin each route edge one by one; these cases
sample the whole shape space the route table covers instead: token counts
from 1 to 40000 (log-uniform, so the small-T column-task route and the row
route both come up), every multiple of 8 from 8 to 16384 as the width, both
weight dtypes, and the plain, residual, per-head, strided and LayerNorm
forms. Every output buffer is filled with NaN first, so an element the
kernels never write fails; every element of y, dx (dh), h and every row's
statistics are compared, and dw (dgamma, dbeta) is checked at the forward's
FP32 statistics and at the FP64 ones, in both modes. The case list comes
from one fixed seed, so a failure names a reproducible case.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import fullsize, synth
from tests.parity import check_dw, check_ln_stats, check_rstd, oracle_rstd32
from tests.test_parity_gpu import (DEV, _announce, dev_bf16, dev_f32, dev_w, filled, host_bits,
                                   nan_f32)

MAX_ELEMS = 1 << 21   # rows x H per case, so the oracle takes well under a second


def _draw_cases(seed: int = 20261203, n: int = 48):
    rng = np.random.default_rng(seed)
    forms = ["plain", "plain", "residual", "heads", "strided", "layernorm"]
    cases = []
    for i in range(n):
        form = forms[int(rng.integers(len(forms)))]
        H = 8 * int(round(math.exp(rng.uniform(0.0, math.log(2048.0)))))
        heads = int(rng.integers(2, 9)) if form in ("heads", "strided") else 1
        t_max = max(1, min(40000, MAX_ELEMS // (H * heads)))
        T = int(round(math.exp(rng.uniform(0.0, math.log(t_max)))))
        T = max(1, min(T, t_max))
        wdt = "bf16" if rng.integers(2) else "f32"
        extra = int(rng.integers(0, 9)) * 8 if form == "strided" else 0
        with_dres = bool(rng.integers(2)) if form == "residual" else False
        cases.append((i, form, T, heads, H, wdt, extra, with_dres))
    return cases


CASES = _draw_cases()


def _ids(c):
    i, form, T, heads, H, wdt, extra, dres = c
    return f"{i}-{form}-T{T}x{heads}x{H}-{wdt}" + (f"-gap{extra}" if extra else "") + \
        ("-dres" if dres else "")


def _rms_case(form, T, heads, H, wdt, extra, with_dres, seed):
    residual = form == "residual"
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=seed, heads=heads, residual=residual,
                    with_dres=with_dres, strided_row=(heads * H + extra) if form == "strided" else 0)
    rows = wl.rows
    w = dev_w(wl.w)
    # ---- forward
    if form in ("plain", "residual"):
        y = filled((rows, H))
        rstd = nan_f32(rows)
        if residual:
            h = filled((rows, H))
            rn.rmsnorm_residual_fwd(dev_bf16(wl.x), dev_bf16(wl.r), w, wl.eps, h=h, y=y, rstd=rstd)
        else:
            rn.rmsnorm_fwd(dev_bf16(wl.x), w, wl.eps, y=y, rstd=rstd)
        torch.cuda.synchronize()
        ybits = host_bits(y)
        src = wl.x
        if residual:
            src = oracle.residual_add(wl.x, wl.r)
            assert np.array_equal(host_bits(h), src), "h = BF16(x + r) not bit-exact"
        rs_got = rstd.cpu().numpy()
    else:
        if form == "strided":
            xbuf = dev_bf16(wl.xbuf)
            xv = xbuf[:, : heads * H].unflatten(1, (heads, H))
        else:
            xv = dev_bf16(wl.x).view(T, heads, H)
        y = filled((T, heads, H))
        rstd = nan_f32(rows).view(T, heads)
        rn.rmsnorm_fwd_strided(xv, w, wl.eps, y=y, rstd=rstd)
        torch.cuda.synchronize()
        ybits = host_bits(y).reshape(rows, H)
        src = wl.x
        rs_got = rstd.cpu().numpy().reshape(-1)
    r64, r32 = oracle_rstd32(src, wl.w.f64, wl.eps)
    check_rstd("rstd", rs_got, r64)
    fullsize.check_y_rows("y", ybits, src, wl.w.f64, wl.eps)
    # ---- backward, fed the oracle's rstd rounded to FP32
    r32_64 = r32.astype(np.float64)
    _, _, dw64 = oracle.bwd(wl.dy, src, r32_64, wl.w.f64, want_dx=False)
    _, _, dw64_i = oracle.bwd(wl.dy, src, r64, wl.w.f64, want_dx=False)
    outs = {}
    for det in (True, False):
        dw = nan_f32(H)
        if form == "plain":
            dx = filled((rows, H))
            rn.rmsnorm_bwd(dev_bf16(wl.dy), dev_bf16(src), dev_f32(r32), w, deterministic=det,
                           dx=dx, dw=dw)
        elif form == "residual":
            dx = filled((rows, H))
            rn.rmsnorm_residual_bwd(dev_bf16(wl.dy), dev_bf16(src), dev_f32(r32), w,
                                    dres=dev_bf16(wl.dres) if with_dres else None,
                                    deterministic=det, dh=dx, dw=dw)
        else:
            dxbuf = filled((T, heads * H + extra))
            dxv = dxbuf[:, : heads * H].unflatten(1, (heads, H))
            rn.rmsnorm_bwd_strided(dev_bf16(wl.dy).view(T, heads, H), xv,
                                   dev_f32(r32).view(T, heads), w, deterministic=det,
                                   dx=dxv, dw=dw)
        torch.cuda.synchronize()
        if form in ("heads", "strided"):
            full = host_bits(dxbuf)
            if extra:
                assert np.all(full[:, heads * H:] == fullsize.SENTINEL), "gap columns written"
            dxbits = np.ascontiguousarray(full[:, : heads * H]).reshape(rows, H)
        else:
            dxbits = host_bits(dx)
        fullsize.check_dx_rows(f"dx det={det}", dxbits, wl.dy, src, r32_64, wl.w.f64,
                               wl.dres if with_dres else None)
        dwh = dw.cpu().numpy()
        check_dw(f"dw det={det} (forward's rstd)", dwh, dw64)
        check_dw(f"dw det={det} (FP64 rstd)", dwh, dw64_i)
        outs[det] = (dxbits, dwh)
    assert np.array_equal(outs[True][0], outs[False][0]), "dx differs between modes"


def _ln_case(T, H, wdt, seed):
    offset = float(np.random.default_rng(seed).uniform(-4.0, 4.0))
    wl = synth.make_ln(T=T, H=H, w_dtype=wdt, seed=seed, offset=offset)
    g, b = dev_w(wl.gamma), dev_w(wl.beta)
    y, mean, rstd = filled((T, H)), nan_f32(T), nan_f32(T)
    rn.layernorm_fwd(dev_bf16(wl.x), g, b, wl.eps, y=y, mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    mu64, rs64, _ = oracle.ln_fwd(wl.x, wl.gamma.f64, wl.beta.f64, wl.eps, want_y=False)
    var64 = np.maximum(1.0 / (rs64 * rs64) - wl.eps, 0.0)
    check_ln_stats("ln", mean.cpu().numpy(), rstd.cpu().numpy(), mu64, rs64, var64)
    fullsize.check_ln_y_rows("y", host_bits(y), wl.x, mu64, rs64, wl.gamma.f64, wl.beta.f64, wl.eps)
    mu32, rs32 = oracle.round_f32(mu64).astype(np.float64), oracle.round_f32(rs64).astype(np.float64)
    _, _, dg64, db64 = oracle.ln_bwd(wl.dy, wl.x, mu32, rs32, wl.gamma.f64, want_dx=False)
    _, _, dg64_i, db64_i = oracle.ln_bwd(wl.dy, wl.x, mu64, rs64, wl.gamma.f64, want_dx=False)
    dxs = []
    for det in (True, False):
        dx, dg, db = filled((T, H)), nan_f32(H), nan_f32(H)
        rn.layernorm_bwd(dev_bf16(wl.dy), dev_bf16(wl.x), dev_f32(mu32), dev_f32(rs32), g,
                         deterministic=det, dx=dx, dgamma=dg, dbeta=db)
        torch.cuda.synchronize()
        dxs.append(host_bits(dx))
        fullsize.check_ln_dx_rows(f"dx det={det}", dxs[-1], wl.dy, wl.x, mu32, rs32, wl.gamma.f64)
        for name, got, r1, r2 in (("dgamma", dg, dg64, dg64_i), ("dbeta", db, db64, db64_i)):
            check_dw(f"{name} det={det} (FP32 statistics)", got.cpu().numpy(), r1)
            check_dw(f"{name} det={det} (FP64 statistics)", got.cpu().numpy(), r2)
    assert np.array_equal(dxs[0], dxs[1]), "dx differs between modes"


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_random_shape(case):
    i, form, T, heads, H, wdt, extra, with_dres = case
    _announce(f"random case {_ids(case)}")
    seed = 1000 + i
    if form == "layernorm":
        _ln_case(T, H, wdt, seed)
    else:
        _rms_case(form, T, heads, H, wdt, extra, with_dres, seed)


def test_case_list_spans_the_routes():
    """The drawn list reaches both backward routes, both weight dtypes, every
    form, widths on both sides of 2048 and partial rows on both sides of the
    8192-row precision switch."""
    forms = {c[1] for c in CASES}
    assert forms == {"plain", "residual", "heads", "strided", "layernorm"}
    assert {c[5] for c in CASES} == {"bf16", "f32"}
    rows = [c[2] * c[3] for c in CASES if c[1] != "layernorm"]
    assert min(rows) <= 64 < max(rows)
    assert any(r > 8192 for r in rows)
    Hs = [c[4] for c in CASES]
    assert min(Hs) < 256 and max(Hs) > 2048
