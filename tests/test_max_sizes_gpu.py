"""The largest shapes the entry points accept, against the FP64 oracle.

* 2^31 - 1 rows of H 8 (the row limit, 34 GB per tensor), plain form;
* 2^31 - 2 rows as 306783378 tokens x 7 heads of H 8 in a strided view with
  a gap (the per-head row split at its 32-bit limit);
* H 16384 (the width limit) over 131072 rows: 2^31 elements per tensor, so
  element offsets pass 2^31;
* the residual form (with dres) and LayerNorm over 2^31 - 1 rows of H 8.

The inputs repeat a period of p rows (p prime to every tile size), built on
the device by repeating p base rows. Every row's outputs then depend on its
row's data only, so they must repeat the base rows' outputs bit for bit: the
oracle checks the p base rows, and a device-side comparison checks that every
later row equals its base row, which covers every element. dw sums every
row: with rows = q*p + m, its FP64 reference is q * (sum over the p base
rows) + (sum over the first m), from two oracle calls, at the rstd the
backward is fed (the forward's, rounded to FP32). The tests on random rows
also hold dw to the budget at the FP64 rstd; that form is left out here,
because its distance from the fed one is the FP32 rounding of each row's
rstd, and with every base row repeated q times those roundings add up in
phase (q * sqrt(p) of them instead of sqrt(rows)): at H 16384 with 61 base
rows they alone reach 1.24 of the budget at a column whose base-row sum
nearly cancels. Every output buffer is filled with NaN first.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import fullsize, synth
from tests.parity import (check_bf16_strict, check_dw, check_dx, check_ln_stats, check_rstd,
                          dx_bound, oracle_rstd32, to_f64)
from tests.test_parity_gpu import DEV, _announce, dev_bf16, dev_f32, dev_w, host_bits

pytestmark = pytest.mark.gpu

ROW_LIMIT = 2 ** 31 - 1


@pytest.fixture(autouse=True)
def _release_cached_memory():
    """Each case needs up to about 150 GB of device memory: hand back what
    earlier tests left in the caching allocator first."""
    _free()
    yield
    _free()


def _periodic(base: torch.Tensor, rows: int) -> torch.Tensor:
    """[rows, W] whose row r is base[r % p] (a fresh contiguous tensor)."""
    p = base.shape[0]
    out = torch.empty((rows,) + tuple(base.shape[1:]), dtype=base.dtype, device=base.device)
    q, m = divmod(rows, p)
    step = max(1, (1 << 26) // max(1, base[0].numel() * p))
    for i in range(0, q, step):
        n = min(step, q - i)
        out[i * p:(i + n) * p].view((n,) + tuple(base.shape)).copy_(base.expand((n,) + tuple(base.shape)))
    if m:
        out[q * p:].copy_(base[:m])
    return out


def _repeats_base(t: torch.Tensor, p: int) -> bool:
    """Every row of t ([rows, ...]) equals row r % p of t itself."""
    rows = t.shape[0]
    base = t[:p]
    q, m = divmod(rows, p)
    step = max(1, (1 << 26) // max(1, base[0].numel() * p))
    for i in range(1, q, step):
        n = min(step, q - i)
        blk = t[i * p:(i + n) * p].reshape((n,) + tuple(base.shape))
        if not torch.equal(blk, base.expand((n,) + tuple(base.shape))):
            return False
    return bool(torch.equal(t[q * p:], t[:m]))


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_case(T, heads, H, wdt, p, gap, seed):
    rows = T * heads
    assert rows <= ROW_LIMIT
    wl = synth.make(T=p, H=H, w_dtype=wdt, seed=seed)
    w = dev_w(wl.w)
    q, m = divmod(rows, p)
    _announce(f"max size T={T} heads={heads} H={H} w={wdt} period={p} gap={gap}: forward")

    # ---- forward
    x_rows = _periodic(dev_bf16(wl.x), rows)
    if heads == 1 and not gap:
        xbuf, xv = None, x_rows
        y = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        rstd = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
        rn.rmsnorm_fwd(xv, w, wl.eps, y=y, rstd=rstd)
    else:
        W = heads * H + gap
        xbuf = torch.zeros((T, W), dtype=torch.bfloat16, device=DEV)
        xv = xbuf[:, : heads * H].unflatten(1, (heads, H))
        xv.copy_(x_rows.view(T, heads, H))
        del x_rows
        _free()
        y = torch.full((T, heads, H), fullsize.SENTINEL, dtype=torch.int16,
                       device=DEV).view(torch.bfloat16)
        rstd = torch.full((T, heads), float("nan"), dtype=torch.float32, device=DEV)
        rn.rmsnorm_fwd_strided(xv, w, wl.eps, y=y, rstd=rstd)
    torch.cuda.synchronize()
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    _, y64 = oracle.fwd(wl.x, wl.w.f64, wl.eps)
    y2 = y.view(rows, H)
    rs1 = rstd.view(rows)
    check_rstd("rstd (base rows)", rs1[:p].cpu().numpy(), r64)
    check_bf16_strict("y (base rows)", host_bits(y2[:p]), y64)
    check_rstd("rstd (last rows)", rs1[rows - m:].cpu().numpy() if m else rs1[:0].cpu().numpy(),
               r64[:m])
    assert _repeats_base(_bits(rs1).view(rows, 1), p), "rstd rows do not repeat the base rows"
    assert _repeats_base(_bits(y2), p), "y rows do not repeat the base rows"
    del y, rstd, y2, rs1
    _free()

    # ---- backward (fed the oracle's FP32 rstd, repeated)
    _announce(f"max size T={T} heads={heads} H={H}: backward")
    dy = _periodic(dev_bf16(wl.dy), rows)
    rs = _periodic(dev_f32(r32).view(p, 1), rows).view(rows)
    dw = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    if xbuf is None:
        dx = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        rn.rmsnorm_bwd(dy, xv, rs, w, deterministic=True, dx=dx, dw=dw)
        torch.cuda.synchronize()
        dx2 = dx
    else:
        dxbuf = torch.full((T, heads * H + gap), fullsize.SENTINEL, dtype=torch.int16,
                           device=DEV).view(torch.bfloat16)
        dxv = dxbuf[:, : heads * H].unflatten(1, (heads, H))
        rn.rmsnorm_bwd_strided(dy.view(T, heads, H), xv, rs.view(T, heads), w, deterministic=True,
                               dx=dxv, dw=dw)
        torch.cuda.synchronize()
        if gap:
            assert bool((dxbuf[:, heads * H:].view(torch.int16) == fullsize.SENTINEL).all()), \
                "gap columns of the dx buffer were written"
        dx2 = dxbuf[:, : heads * H].reshape(rows, H)
    r32_64 = r32.astype(np.float64)
    dx64, c64, dw_all = oracle.bwd(wl.dy, wl.x, r32_64, wl.w.f64)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32_64, c64, H)
    check_dx("dx (base rows)", host_bits(dx2[:p]), dx64, E)
    assert _repeats_base(_bits(dx2), p), "dx rows do not repeat the base rows"
    if m:
        _, _, dw_m = oracle.bwd(wl.dy[:m], wl.x[:m], r32_64[:m], wl.w.f64, want_dx=False)
    else:
        dw_m = np.zeros(H)
    check_dw("dw (the fed rstd)", dw.cpu().numpy(), q * dw_all + dw_m)
    del dy, rs, dw, dx2, xv
    if xbuf is None:
        del dx
    else:
        del dxbuf, dxv, xbuf
    _free()


def test_row_limit_plain():
    """2^31 - 1 rows of H 8: the largest row count the entry points accept."""
    _check_case(T=ROW_LIMIT, heads=1, H=8, wdt="bf16", p=4099, gap=0, seed=71)


def test_row_limit_strided_heads():
    """306783378 tokens x 7 heads of H 8 (2^31 - 2 rows) in a strided view with
    an 8-element gap per token: the per-head row split at its 32-bit limit."""
    _check_case(T=ROW_LIMIT // 7, heads=7, H=8, wdt="f32", p=4093, gap=8, seed=72)


def test_width_limit_past_2_31_elements():
    """H 16384 over 131072 rows: 2^31 elements per tensor."""
    _check_case(T=131072, heads=1, H=16384, wdt="bf16", p=61, gap=0, seed=73)


def test_row_limit_residual():
    """The fused residual form over 2^31 - 1 rows of H 8, with dres."""
    rows, H, p = ROW_LIMIT, 8, 4091
    q, m = divmod(rows, p)
    wl = synth.make(T=p, H=H, w_dtype="bf16", seed=74, residual=True, with_dres=True)
    w = dev_w(wl.w)
    _announce(f"max size residual rows={rows} H={H} period={p}: forward")
    x = _periodic(dev_bf16(wl.x), rows)
    r = _periodic(dev_bf16(wl.r), rows)
    h = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rstd = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    rn.rmsnorm_residual_fwd(x, r, w, wl.eps, h=h, y=y, rstd=rstd)
    torch.cuda.synchronize()
    del x, r
    h_ref = oracle.residual_add(wl.x, wl.r)
    assert np.array_equal(host_bits(h[:p]), h_ref), "h (base rows) not bit-exact"
    r64, r32 = oracle_rstd32(h_ref, wl.w.f64, wl.eps)
    _, y64 = oracle.fwd(h_ref, wl.w.f64, wl.eps)
    check_rstd("rstd (base rows)", rstd[:p].cpu().numpy(), r64)
    check_bf16_strict("y (base rows)", host_bits(y[:p]), y64)
    for name, t in (("h", _bits(h)), ("y", _bits(y)), ("rstd", _bits(rstd).view(rows, 1))):
        assert _repeats_base(t, p), f"{name} rows do not repeat the base rows"
    del h, y, rstd
    _free()

    _announce(f"max size residual rows={rows} H={H}: backward")
    hin = _periodic(dev_bf16(h_ref), rows)
    dy = _periodic(dev_bf16(wl.dy), rows)
    dres = _periodic(dev_bf16(wl.dres), rows)
    rs = _periodic(dev_f32(r32).view(p, 1), rows).view(rows)
    dh = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dw = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    rn.rmsnorm_residual_bwd(dy, hin, rs, w, dres=dres, deterministic=True, dh=dh, dw=dw)
    torch.cuda.synchronize()
    r32_64 = r32.astype(np.float64)
    dx64, c64, dw_all = oracle.bwd(wl.dy, h_ref, r32_64, wl.w.f64)
    dres64 = to_f64(wl.dres)
    E = dx_bound(to_f64(h_ref), to_f64(wl.dy), wl.w.f64, r32_64, c64, H, dres64)
    check_dx("dh (base rows)", host_bits(dh[:p]), dx64 + dres64, E)
    assert _repeats_base(_bits(dh), p), "dh rows do not repeat the base rows"
    _, _, dw_m = oracle.bwd(wl.dy[:m], h_ref[:m], r32_64[:m], wl.w.f64, want_dx=False)
    check_dw("dw (the fed rstd)", dw.cpu().numpy(), q * dw_all + dw_m)
    del hin, dy, dres, rs, dh, dw
    _free()


def test_row_limit_layernorm():
    """LayerNorm over 2^31 - 1 rows of H 8, gamma and beta FP32."""
    rows, H, p = ROW_LIMIT, 8, 4079
    q, m = divmod(rows, p)
    wl = synth.make_ln(T=p, H=H, w_dtype="f32", seed=75, offset=1.5)
    g, b = dev_w(wl.gamma), dev_w(wl.beta)
    _announce(f"max size layernorm rows={rows} H={H} period={p}: forward")
    x = _periodic(dev_bf16(wl.x), rows)
    y = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    mean = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    rstd = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    rn.layernorm_fwd(x, g, b, wl.eps, y=y, mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    mu64, rs64, _ = oracle.ln_fwd(wl.x, wl.gamma.f64, wl.beta.f64, wl.eps, want_y=False)
    var64 = np.maximum(1.0 / (rs64 * rs64) - wl.eps, 0.0)
    check_ln_stats("ln (base rows)", mean[:p].cpu().numpy(), rstd[:p].cpu().numpy(), mu64, rs64, var64)
    fullsize.check_ln_y_rows("y (base rows)", host_bits(y[:p]), wl.x, mu64, rs64, wl.gamma.f64,
                             wl.beta.f64, wl.eps)
    for name, t in (("y", _bits(y)), ("mean", _bits(mean).view(rows, 1)),
                    ("rstd", _bits(rstd).view(rows, 1))):
        assert _repeats_base(t, p), f"{name} rows do not repeat the base rows"
    del y, mean, rstd
    _free()

    _announce(f"max size layernorm rows={rows} H={H}: backward")
    mu32 = oracle.round_f32(mu64).astype(np.float64)
    rs32 = oracle.round_f32(rs64).astype(np.float64)
    dy = _periodic(dev_bf16(wl.dy), rows)
    mu_d = _periodic(dev_f32(mu32).view(p, 1), rows).view(rows)
    rs_d = _periodic(dev_f32(rs32).view(p, 1), rows).view(rows)
    dx = torch.full((rows, H), fullsize.SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dg = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    rn.layernorm_bwd(dy, x, mu_d, rs_d, g, deterministic=True, dx=dx, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    fullsize.check_ln_dx_rows("dx (base rows)", host_bits(dx[:p]), wl.dy, wl.x, mu32, rs32,
                              wl.gamma.f64)
    assert _repeats_base(_bits(dx), p), "dx rows do not repeat the base rows"
    _, _, dg_all, db_all = oracle.ln_bwd(wl.dy, wl.x, mu32, rs32, wl.gamma.f64, want_dx=False)
    _, _, dg_m, db_m = oracle.ln_bwd(wl.dy[:m], wl.x[:m], mu32[:m], rs32[:m], wl.gamma.f64,
                                     want_dx=False)
    check_dw("dgamma (the fed statistics)", dg.cpu().numpy(), q * dg_all + dg_m)
    check_dw("dbeta", db.cpu().numpy(), q * db_all + db_m)
    del x, dy, mu_d, rs_d, dx, dg, db
    _free()
