"""Seeded random shapes through the public RMSNorm and LayerNorm entry
points, against the FP64 oracle.

The hand-picked shapes elsewhere pin each route edge one by one; these cases
sample the whole shape space the route table covers instead: token counts
from 1 to 40000 (log-uniform, so the small-T column-task route and the row
route both come up), every multiple of 8 from 8 to 16384 as the width, both
weight dtypes, and the plain, residual (contiguous and over views),
per-head, strided, recompute-backward, allocation-free and LayerNorm forms. Every output buffer is filled with NaN first, so an element the
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
from tests.parity import (check_dw, check_dx, check_ln_stats, check_rstd, dx_bound,
                          oracle_rstd32, to_f64)
from tests.test_parity_gpu import (DEV, _announce, dev_bf16, dev_f32, dev_w, filled, host_bits,
                                   nan_f32)

MAX_ELEMS = 1 << 21   # rows x H per case, so the oracle takes well under a second


def _draw_cases(seed: int = 20261203, n: int = 72):
    rng = np.random.default_rng(seed)
    forms = ["plain", "plain", "residual", "residual_views", "heads", "strided", "recompute",
             "noalloc", "layernorm"]
    cases = []
    for i in range(n):
        form = forms[int(rng.integers(len(forms)))]
        H = 8 * int(round(math.exp(rng.uniform(0.0, math.log(2048.0)))))
        viewed = form in ("heads", "strided", "residual_views", "recompute", "noalloc")
        heads = int(rng.integers(1 if form != "heads" else 2, 9)) if viewed else 1
        t_max = max(1, min(40000, MAX_ELEMS // (H * heads)))
        T = int(round(math.exp(rng.uniform(0.0, math.log(t_max)))))
        T = max(1, min(T, t_max))
        wdt = "bf16" if rng.integers(2) else "f32"
        extra = int(rng.integers(0, 9)) * 8 if viewed and form != "heads" else 0
        with_dres = bool(rng.integers(2)) if form in ("residual", "residual_views") else False
        cases.append((i, form, T, heads, H, wdt, extra, with_dres))
    return cases


CASES = _draw_cases()


def _ids(c):
    i, form, T, heads, H, wdt, extra, dres = c
    return f"{i}-{form}-T{T}x{heads}x{H}-{wdt}" + (f"-gap{extra}" if extra else "") + \
        ("-dres" if dres else "")


def _rms_case(form, T, heads, H, wdt, extra, with_dres, seed):
    residual = form == "residual"
    strided = form in ("strided", "noalloc")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=seed, heads=heads, residual=residual,
                    with_dres=with_dres, strided_row=(heads * H + extra) if strided else 0)
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
        if strided:
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
            call = rn.rmsnorm_bwd_strided_noalloc if form == "noalloc" else rn.rmsnorm_bwd_strided
            call(dev_bf16(wl.dy).view(T, heads, H), xv, dev_f32(r32).view(T, heads), w,
                 deterministic=det, dx=dxv, dw=dw)
        torch.cuda.synchronize()
        if form in ("heads", "strided", "noalloc"):
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


def _wide(bits, T, heads, H, gap):
    """A [T, heads*H + gap] buffer: NaN fill, with `bits` (rows of H) in the
    first heads*H columns if given; returns (buffer, [T, heads, H] view)."""
    buf = filled((T, heads * H + gap))
    view = buf[:, : heads * H].unflatten(1, (heads, H))
    if bits is not None:
        view.copy_(dev_bf16(bits).view(T, heads, H))
    return buf, view


def _rows_of(buf, T, heads, H, gap):
    full = host_bits(buf)
    if gap:
        assert np.all(full[:, heads * H:] == fullsize.SENTINEL), "gap columns written"
    return np.ascontiguousarray(full[:, : heads * H]).reshape(T * heads, H)


def _residual_views_case(T, heads, H, wdt, gap, with_dres, seed):
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=seed, heads=heads, residual=True,
                    with_dres=with_dres)
    w = dev_w(wl.w)
    _, xv = _wide(wl.x, T, heads, H, gap)
    _, rv = _wide(wl.r, T, heads, H, gap)
    hb, hv = _wide(None, T, heads, H, gap)
    yb, yv = _wide(None, T, heads, H, gap)
    rstd = nan_f32(T * heads).view(T, heads)
    rn.rmsnorm_residual_fwd_strided(xv, rv, w, wl.eps, h=hv, y=yv, rstd=rstd)
    torch.cuda.synchronize()
    h_ref = oracle.residual_add(wl.x, wl.r)
    assert np.array_equal(_rows_of(hb, T, heads, H, gap), h_ref), "h = BF16(x + r) not bit-exact"
    r64, r32 = oracle_rstd32(h_ref, wl.w.f64, wl.eps)
    check_rstd("rstd", rstd.cpu().numpy().reshape(-1), r64)
    fullsize.check_y_rows("y", _rows_of(yb, T, heads, H, gap), h_ref, wl.w.f64, wl.eps)
    r32_64 = r32.astype(np.float64)
    _, _, dw64 = oracle.bwd(wl.dy, h_ref, r32_64, wl.w.f64, want_dx=False)
    _, _, dw64_i = oracle.bwd(wl.dy, h_ref, r64, wl.w.f64, want_dx=False)
    _, dyv = _wide(wl.dy, T, heads, H, gap)
    _, hin = _wide(h_ref, T, heads, H, gap)
    drv = _wide(wl.dres, T, heads, H, gap)[1] if with_dres else None
    outs = []
    for det in (True, False):
        dhb, dhv = _wide(None, T, heads, H, gap)
        dw = nan_f32(H)
        rn.rmsnorm_residual_bwd_strided(dyv, hin, dev_f32(r32).view(T, heads), w, dres=drv,
                                        deterministic=det, dh=dhv, dw=dw)
        torch.cuda.synchronize()
        outs.append(_rows_of(dhb, T, heads, H, gap))
        fullsize.check_dx_rows(f"dh det={det}", outs[-1], wl.dy, h_ref, r32_64, wl.w.f64,
                               wl.dres if with_dres else None)
        check_dw(f"dw det={det} (forward's rstd)", dw.cpu().numpy(), dw64)
        check_dw(f"dw det={det} (FP64 rstd)", dw.cpu().numpy(), dw64_i)
    assert np.array_equal(outs[0], outs[1]), "dh differs between modes"


def _recompute_case(T, heads, H, wdt, gap, seed):
    """The backward that recomputes rstd from x: dx within one ulp, or ulp
    plus the plain bound widened by the effect of a one-ulp FP32 difference
    in rstd (d(dx)/d(rstd) = g - 3 xhat c)."""
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=seed, heads=heads)
    w = dev_w(wl.w)
    _, xv = _wide(wl.x, T, heads, H, gap)
    _, dyv = _wide(wl.dy, T, heads, H, gap)
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    r32_64 = r32.astype(np.float64)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32_64, wl.w.f64)
    _, _, dw64_i = oracle.bwd(wl.dy, wl.x, r64, wl.w.f64, want_dx=False)
    x64, dy64 = to_f64(wl.x), to_f64(wl.dy)
    E = dx_bound(x64, dy64, wl.w.f64, r32_64, c64, H)
    g = dy64 * wl.w.f64[None, :]
    E = E + 2.0 ** -23 * r32_64[:, None] * (np.abs(g) + 3.0 * np.abs(x64 * r32_64[:, None] * c64[:, None]))
    outs = []
    for det in (True, False):
        dxb, dxv = _wide(None, T, heads, H, gap)
        dw = nan_f32(H)
        rn.rmsnorm_bwd_recompute(dyv, xv, w, wl.eps, deterministic=det, dx=dxv, dw=dw)
        torch.cuda.synchronize()
        outs.append(_rows_of(dxb, T, heads, H, gap))
        check_dx(f"dx det={det}", outs[-1], dx64, E)
        check_dw(f"dw det={det} (forward's rstd)", dw.cpu().numpy(), dw64)
        check_dw(f"dw det={det} (FP64 rstd)", dw.cpu().numpy(), dw64_i)
    assert np.array_equal(outs[0], outs[1]), "dx differs between modes"


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
    elif form == "residual_views":
        _residual_views_case(T, heads, H, wdt, extra, with_dres, seed)
    elif form == "recompute":
        _recompute_case(T, heads, H, wdt, extra, seed)
    else:
        _rms_case(form, T, heads, H, wdt, extra, with_dres, seed)


def test_case_list_spans_the_routes():
    """The drawn list reaches both backward routes, both weight dtypes, every
    form, widths on both sides of 2048 and partial rows on both sides of the
    8192-row precision switch."""
    forms = {c[1] for c in CASES}
    assert forms == {"plain", "residual", "residual_views", "heads", "strided", "recompute",
                     "noalloc", "layernorm"}
    assert {c[5] for c in CASES} == {"bf16", "f32"}
    rows = [c[2] * c[3] for c in CASES if c[1] != "layernorm"]
    assert min(rows) <= 64 < max(rows)
    assert any(r > 8192 for r in rows)
    Hs = [c[4] for c in CASES]
    assert min(Hs) < 256 and max(Hs) > 2048
