"""Parity of the HIP path (through the C ABI) with the FP64 oracle.

Small shapes span several blocks, ragged rows (H not a multiple of the lane
count), both weight dtypes, both modes, the small-T column-task route and
the large-T row route. Full-size cases run each workload the method is
quoted on, in the same launch configuration the benchmark times, and check
every element of y and dx (dh, h), every row's rstd, every column of dw, and
bit-reproducibility of deterministic dw; outputs are filled with a NaN
pattern first, so an element the kernels never write fails.

The backward is fed the oracle's rstd rounded to FP32 (never the GPU
forward's), so no oracle input comes from the HIP path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import fullsize, synth
from tests.parity import (check_bf16_strict, check_dw, check_dx, check_rstd, dx_bound,
                          oracle_rstd32, to_f64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def dev_w(w: synth.Weight) -> torch.Tensor:
    if w.dtype == "bf16":
        return dev_bf16(w.bits)
    return torch.from_numpy(w.f32.copy()).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def _announce(msg: str) -> None:
    print(msg, flush=True)


# ------------------------------------------------------------ small shapes

SMALL = [
    (1, 8, "f32"), (3, 24, "bf16"), (64, 256, "f32"), (65, 256, "f32"), (37, 4096, "bf16"),
    (300, 2048, "f32"), (129, 6144, "bf16"), (70, 1032, "bf16"), (257, 16384, "bf16"),
    (1000, 512, "f32"), (2049, 1536, "bf16"), (5, 16384, "f32"), (40, 6144, "f32"),
    (9000, 128, "bf16"), (700, 5120, "f32"),
    # ragged for the multi-row launch shapes (4 rows per iteration at H 2048,
    # 2 row groups at H 5120), FP64 partials above 8192 rows
    (303, 2048, "bf16"), (701, 5120, "bf16"), (10007, 2048, "f32"),
    # widths between 2048 and 4096: three row groups of 320 lanes per block
    # up to H 2560, two of 384 or 448 lanes above
    (333, 2304, "bf16"), (1001, 2560, "f32"), (97, 3072, "bf16"), (129, 3584, "f32"),
    # more small-T column-task shapes: ragged widths, a single column chunk,
    # narrow rows, and T just below the row route
    (17, 136, "bf16"), (32, 512, "f32"), (33, 512, "bf16"), (64, 8, "f32"), (2, 520, "f32"),
]


@pytest.mark.parametrize("T,H,wdt", SMALL)
def test_fwd_small(T, H, wdt):
    _announce(f"fwd T={T} H={H} w={wdt}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + H)
    y, rstd = rn.rmsnorm_fwd(dev_bf16(wl.x), dev_w(wl.w), wl.eps)
    torch.cuda.synchronize()
    r64, y64 = oracle.fwd(wl.x, wl.w.f64, wl.eps)
    check_rstd("rstd", rstd.cpu().numpy(), r64)
    check_bf16_strict("y", host_bits(y), y64)


def _bwd_case(wl, det, rstd32):
    x, dy, w = dev_bf16(wl.x), dev_bf16(wl.dy), dev_w(wl.w)
    rs = dev_f32(rstd32)
    dx, dw = rn.rmsnorm_bwd(dy, x, rs, w, deterministic=det)
    torch.cuda.synchronize()
    return host_bits(dx), dw.cpu().numpy()


@pytest.mark.parametrize("T,H,wdt", SMALL)
def test_bwd_small(T, H, wdt):
    _announce(f"bwd T={T} H={H} w={wdt}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=3 * T + H)
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    r32_64 = r32.astype(np.float64)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32_64, wl.w.f64)
    _, _, dw64_i = oracle.bwd(wl.dy, wl.x, r64, wl.w.f64, want_dx=False)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32_64, c64, H)
    dx_det, dw_det = _bwd_case(wl, True, r32)
    check_dx("dx det", dx_det, dx64, E)
    check_dw("dw det (forward's rstd)", dw_det, dw64)
    check_dw("dw det (FP64 rstd)", dw_det, dw64_i)
    dx_nd, dw_nd = _bwd_case(wl, False, r32)
    assert np.array_equal(dx_nd, dx_det), "dx differs between modes"
    check_dw("dw non-det", dw_nd, dw64)
    for _ in range(3):
        dx2, dw2 = _bwd_case(wl, True, r32)
        assert np.array_equal(dw2.view(np.uint32), dw_det.view(np.uint32)), "det dw not reproducible"
        assert np.array_equal(dx2, dx_det)


@pytest.mark.parametrize("T,H,wdt,with_dres", [(64, 6144, "bf16", True), (333, 6144, "bf16", True),
                                                (333, 6144, "f32", False), (100, 256, "f32", True),
                                                (50, 256, "f32", True), (7, 512, "bf16", False)])
def test_residual_small(T, H, wdt, with_dres):
    _announce(f"residual T={T} H={H} w={wdt} dres={with_dres}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + 7, residual=True, with_dres=with_dres)
    h, y, rstd = rn.rmsnorm_residual_fwd(dev_bf16(wl.x), dev_bf16(wl.r), dev_w(wl.w), wl.eps)
    torch.cuda.synchronize()
    h_ref = oracle.residual_add(wl.x, wl.r)
    assert np.array_equal(host_bits(h), h_ref), "h = BF16(x + r) not bit-exact"
    r64, y64 = oracle.fwd(h_ref, wl.w.f64, wl.eps)
    check_rstd("rstd", rstd.cpu().numpy(), r64)
    check_bf16_strict("y", host_bits(y), y64)
    r32 = oracle.round_f32(r64)
    dx64, c64, dw64 = oracle.bwd(wl.dy, h_ref, r32.astype(np.float64), wl.w.f64)
    dres64 = to_f64(wl.dres) if with_dres else None
    dh64 = dx64 + (dres64 if with_dres else 0.0)
    E = dx_bound(to_f64(h_ref), to_f64(wl.dy), wl.w.f64, r32.astype(np.float64), c64, H, dres64)
    outs = []
    for det in (True, False):
        dh, dw = rn.rmsnorm_residual_bwd(dev_bf16(wl.dy), dev_bf16(h_ref), dev_f32(r32), dev_w(wl.w),
                                         dres=dev_bf16(wl.dres) if with_dres else None,
                                         deterministic=det)
        torch.cuda.synchronize()
        outs.append(host_bits(dh))
        check_dx(f"dh det={det}", outs[-1], dh64, E)
        check_dw(f"dw det={det}", dw.cpu().numpy(), dw64)
    assert np.array_equal(outs[0], outs[1])


def _strided_case(T, heads, H, row, seed):
    wl = synth.make(T=T, H=H, w_dtype="f32", seed=seed, heads=heads, strided_row=row)
    xbuf = dev_bf16(wl.xbuf)
    xview = xbuf[:, : heads * H].unflatten(1, (heads, H))
    return wl, xbuf, xview


@pytest.mark.parametrize("T,heads,H,row", [(300, 24, 256, 8192), (50, 4, 256, 1024), (7, 3, 512, 2048)])
def test_strided_heads_small(T, heads, H, row):
    _announce(f"strided T={T} heads={heads} H={H} row={row}")
    wl, xbuf, xview = _strided_case(T, heads, H, row, seed=T + heads)
    w = dev_w(wl.w)
    y, rstd = rn.rmsnorm_fwd_strided(xview, w, wl.eps)
    torch.cuda.synchronize()
    r64, y64 = oracle.fwd(wl.x, wl.w.f64, wl.eps)
    check_rstd("rstd", rstd.cpu().numpy().reshape(-1), r64)
    check_bf16_strict("y", host_bits(y).reshape(-1, H), y64)
    r32 = oracle.round_f32(r64)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32.astype(np.float64), c64, H)
    dy = dev_bf16(wl.dy).view(T, heads, H)
    rs = dev_f32(r32).view(T, heads)
    sentinel = 0x7FC0
    dxbuf = torch.full((T, row), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dxview = dxbuf[:, : heads * H].unflatten(1, (heads, H))
    for det in (True, False):
        _, dw = rn.rmsnorm_bwd_strided(dy, xview, rs, w, deterministic=det, dx=dxview)
        torch.cuda.synchronize()
        full = host_bits(dxbuf)
        assert np.all(full[:, heads * H:] == sentinel), "gap columns of the dx buffer were written"
        check_dx(f"dx det={det}", np.ascontiguousarray(full[:, : heads * H]).reshape(-1, H), dx64, E)
        check_dw(f"dw det={det}", dw.cpu().numpy(), dw64)
    # strided and contiguous inputs give the same bits (row-local outputs,
    # same deterministic partition)
    xc = dev_bf16(wl.x).view(T, heads, H)
    yc, rc = rn.rmsnorm_fwd_strided(xc, w, wl.eps)
    dxc, dwc = rn.rmsnorm_bwd_strided(dy, xc, rs, w, deterministic=True)
    _, dws = rn.rmsnorm_bwd_strided(dy, xview, rs, w, deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(yc.view(torch.int16), y.view(torch.int16))
    assert torch.equal(rc, rstd)
    assert np.array_equal(host_bits(dxc).reshape(-1, H),
                          np.ascontiguousarray(host_bits(dxbuf)[:, : heads * H]).reshape(-1, H))
    assert torch.equal(dwc.view(torch.int32), dws.view(torch.int32))


def test_zero_rows_and_errors():
    w = torch.ones(64, dtype=torch.float32, device=DEV)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    y, rstd = rn.rmsnorm_fwd(x, w)
    dx, dw = rn.rmsnorm_bwd(x, x, rstd, w, deterministic=True, dw=torch.full((64,), 7.0, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(dw == 0)
    with pytest.raises(rn.RMSNormError):
        rn.rmsnorm_fwd(torch.zeros(4, 60, dtype=torch.bfloat16, device=DEV),
                       torch.ones(60, device=DEV))
    with pytest.raises(rn.RMSNormError):
        xx = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
        rn.rmsnorm_fwd(xx, w, eps=-1.0)


def test_atomic_route_with_dirty_workspace():
    """The atomic route clears its own accumulator: a workspace full of
    garbage (as the two-stage route leaves it) gives the same budget."""
    wl = synth.make(T=4096, H=1024, w_dtype="bf16", seed=5)
    _, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    _, _, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64, want_dx=False)
    try:
        rn.rmsnorm_route_override("bwd", kind=3)
        need = rn.rmsnorm_bwd_workspace_bytes(4096, 1024, torch.bfloat16, False)
        ws = torch.full((need + 256,), 0x5A, dtype=torch.uint8, device=DEV)
        ws = ws[(-ws.data_ptr()) % 256:]
        for _ in range(3):
            _, dw = rn.rmsnorm_bwd(dev_bf16(wl.dy), dev_bf16(wl.x), dev_f32(r32), dev_w(wl.w),
                                   deterministic=False, workspace=ws)
            torch.cuda.synchronize()
            check_dw("dw non-det atomic", dw.cpu().numpy(), dw64)
            ws.fill_(0x5A)
    finally:
        rn.rmsnorm_route_override("bwd")


# --------------------------------------------------------- full-size cases

def filled(shape, device=DEV) -> torch.Tensor:
    """A BF16 buffer holding the NaN fill pattern in every element."""
    return torch.full(shape, fullsize.SENTINEL, dtype=torch.int16, device=device).view(torch.bfloat16)


def nan_f32(n: int) -> torch.Tensor:
    return torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("name", list(synth.CONFIGS) + list(synth.WIDTH_CONFIGS))
def test_full_size_config(name):
    """Every element of y, dx (dh) and h of the full-size workload, in the
    launch configuration the benchmark times, against the oracle; every
    row's rstd and every column of dw; deterministic dw bit-identical over
    10 runs; dx identical between the modes. Outputs start as NaN patterns."""
    _announce(f"full-size {name}: generating")
    wl = synth.config(name, seed=0)
    rows, H = wl.rows, wl.H
    w = dev_w(wl.w)
    res = wl.r is not None
    shape3 = (wl.T, wl.heads, H)
    # ---------------- forward on the GPU
    if res:
        h = filled((rows, H))
        y = filled((rows, H))
        h, y, rstd = rn.rmsnorm_residual_fwd(dev_bf16(wl.x), dev_bf16(wl.r), w, wl.eps, h=h, y=y,
                                             rstd=nan_f32(rows))
        torch.cuda.synchronize()
        x_in = oracle.residual_add(wl.x, wl.r)
        assert np.array_equal(host_bits(h), x_in), "h not bit-exact"
        del h
    elif wl.xbuf is not None:
        xbuf = dev_bf16(wl.xbuf)
        xd = xbuf[:, : wl.heads * H].unflatten(1, (wl.heads, H))
        y, rstd = rn.rmsnorm_fwd_strided(xd, w, wl.eps, y=filled(shape3), rstd=nan_f32(rows))
        x_in = wl.x
    elif wl.heads > 1:
        xd = dev_bf16(wl.x).view(shape3)
        y, rstd = rn.rmsnorm_fwd_strided(xd, w, wl.eps, y=filled(shape3), rstd=nan_f32(rows))
        x_in = wl.x
    else:
        xd = dev_bf16(wl.x)
        y, rstd = rn.rmsnorm_fwd(xd, w, wl.eps, y=filled((rows, H)), rstd=nan_f32(rows))
        x_in = wl.x
    torch.cuda.synchronize()
    _announce(f"full-size {name}: oracle forward, all {rows} rows")
    r64, r32 = oracle_rstd32(x_in, wl.w.f64, wl.eps)
    check_rstd("rstd (all rows)", rstd.cpu().numpy().reshape(-1), r64)
    ybits = host_bits(y).reshape(rows, H)
    del y
    fullsize.check_y_rows("y", ybits, x_in, wl.w.f64, wl.eps)
    del ybits
    # ---------------- backward on the GPU, fed the oracle's FP32 rstd
    rs = dev_f32(r32)
    dy = dev_bf16(wl.dy)
    r32_64 = r32.astype(np.float64)
    _announce(f"full-size {name}: oracle dw over all rows, both rstd forms")
    _, _, dw64 = oracle.bwd(wl.dy, x_in, r32_64, wl.w.f64, want_dx=False)
    _, _, dw64_i = oracle.bwd(wl.dy, x_in, r64, wl.w.f64, want_dx=False)
    if res:
        x_dev = dev_bf16(x_in)

    def run_bwd(det):
        dwt = nan_f32(H)
        if res:
            dx, dw = rn.rmsnorm_residual_bwd(dy, x_dev, rs, w,
                                             dres=dev_bf16(wl.dres) if wl.dres is not None else None,
                                             deterministic=det, dh=filled((rows, H)), dw=dwt)
            torch.cuda.synchronize()
            return host_bits(dx).reshape(rows, H), dw.cpu().numpy()
        if wl.xbuf is not None:
            dxbuf = filled(wl.xbuf.shape)
            dxv = dxbuf[:, : wl.heads * H].unflatten(1, (wl.heads, H))
            _, dw = rn.rmsnorm_bwd_strided(dy.view(shape3), xd, rs.view(wl.T, wl.heads), w,
                                           deterministic=det, dx=dxv, dw=dwt)
            torch.cuda.synchronize()
            full = host_bits(dxbuf)
            assert np.all(full[:, wl.heads * H:] == fullsize.SENTINEL), "gap columns written"
            return np.ascontiguousarray(full[:, : wl.heads * H]).reshape(rows, H), dw.cpu().numpy()
        if wl.heads > 1:
            dx, dw = rn.rmsnorm_bwd_strided(dy.view(shape3), xd, rs.view(wl.T, wl.heads), w,
                                            deterministic=det, dx=filled(shape3), dw=dwt)
            torch.cuda.synchronize()
            return host_bits(dx).reshape(rows, H), dw.cpu().numpy()
        dx, dw = rn.rmsnorm_bwd(dy, xd, rs, w, deterministic=det, dx=filled((rows, H)), dw=dwt)
        torch.cuda.synchronize()
        return host_bits(dx), dw.cpu().numpy()

    det_dx_bits = None
    det_dw_bits = None
    for det in (True, False):
        _announce(f"full-size {name}: backward det={det}")
        dxb, dwn = run_bwd(det)
        f2 = check_dw(f"dw det={det} (forward's rstd)", dwn, dw64)
        f1 = check_dw(f"dw det={det} (FP64 rstd)", dwn, dw64_i)
        if det:
            n_ex = fullsize.check_dx_rows("dx det", dxb, wl.dy, x_in, r32_64, wl.w.f64,
                                          wl.dres if res else None)
            _announce(f"  dx all rows: exempted={n_ex}; dw worst/budget={f2:.4f} "
                      f"(fp64-rstd form {f1:.4f})")
            det_dx_bits, det_dw_bits = dxb, dwn.view(np.uint32).copy()
        else:
            assert np.array_equal(dxb, det_dx_bits), "dx differs between modes"
            _announce(f"  non-det: dx identical to det; dw worst/budget={f2:.4f} ({f1:.4f})")
        del dxb
    del det_dx_bits
    # deterministic dw: bit-identical over 10 runs
    for i in range(10):
        _, dwn = run_bwd(True)
        assert np.array_equal(dwn.view(np.uint32), det_dw_bits), f"deterministic dw changed on run {i}"
    # non-deterministic dw: inside the budget on every run
    for i in range(3):
        _, dwn = run_bwd(False)
        check_dw(f"dw non-det run {i}", dwn, dw64)


# ------------------------------------------------- non-default launch shapes

VARIANTS = [
    # (T, H, w dtype, op, knobs)
    (3000, 256, "f32", "fwd", dict(vec_per_lane=1, unroll=4)),
    (3000, 256, "f32", "fwd", dict(vec_per_lane=1, unroll=1, rows_per_block=2)),
    (777, 2048, "bf16", "fwd", dict(vec_per_lane=4, unroll=1)),
    (777, 4096, "bf16", "fwd", dict(vec_per_lane=4)),
    (777, 4096, "f32", "fwd", dict(vec_per_lane=1, rows_per_block=2, blocks_per_cu=1)),
    (3000, 256, "f32", "bwd", dict(vec_per_lane=1, unroll=4, blocks_per_cu=2)),
    (3000, 256, "bf16", "bwd", dict(vec_per_lane=1, unroll=1, rows_per_block=4)),
    (777, 2048, "f32", "bwd", dict(vec_per_lane=2, rows_per_block=2, partial_f64=1)),
    (777, 4096, "bf16", "bwd", dict(vec_per_lane=2, blocks_per_cu=2, partial_f64=2)),
    (5000, 6144, "bf16", "bwd", dict(vec_per_lane=1, blocks_per_cu=2)),
    (777, 4096, "bf16", "fwd", dict(vec_per_lane=1, unroll=8)),
    (777, 6144, "bf16", "fwd", dict(vec_per_lane=2, unroll=4, rows_per_block=1)),
    (777, 4096, "bf16", "bwd", dict(vec_per_lane=1, unroll=4, rows_per_block=1)),
    (777, 4096, "bf16", "bwd", dict(vec_per_lane=1, unroll=2, rows_per_block=1)),
    (3000, 2048, "f32", "bwd", dict(vec_per_lane=2, unroll=1, rows_per_block=4)),
    (5000, 2048, "f32", "bwd", dict(vec_per_lane=1, unroll=4, rows_per_block=2)),
    (1000, 6144, "bf16", "bwd", dict(vec_per_lane=2, unroll=2)),
    (2500, 1024, "f32", "bwd", dict(kind=3)),  # atomic finalise, non-deterministic calls
    (300, 256, "f32", "bwd", dict(kind=3, vec_per_lane=1, unroll=2)),
]


@pytest.mark.parametrize("T,H,wdt,op,knobs", VARIANTS)
def test_route_variants(T, H, wdt, op, knobs):
    _announce(f"variant {op} T={T} H={H} w={wdt} {knobs}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + H + 1)
    try:
        rn.rmsnorm_route_override(op, **knobs)
        if op == "fwd":
            y, rstd = rn.rmsnorm_fwd(dev_bf16(wl.x), dev_w(wl.w), wl.eps)
            torch.cuda.synchronize()
            r64, y64 = oracle.fwd(wl.x, wl.w.f64, wl.eps)
            check_rstd("rstd", rstd.cpu().numpy(), r64)
            check_bf16_strict("y", host_bits(y), y64)
            return
        _, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
        r32_64 = r32.astype(np.float64)
        dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32_64, wl.w.f64)
        E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32_64, c64, H)
        det = "kind" not in knobs
        outs = []
        for _ in range(3):
            dx, dw = _bwd_case(wl, det, r32)
            check_dx("dx", dx, dx64, E)
            check_dw("dw", dw, dw64)
            outs.append((dx, dw))
        if det:
            assert all(np.array_equal(o[1].view(np.uint32), outs[0][1].view(np.uint32)) for o in outs)
        else:
            # same row layout, deterministic mode: dx bit-identical
            dx_det, _ = _bwd_case(wl, True, r32)
            assert np.array_equal(outs[0][0], dx_det)
    finally:
        rn.rmsnorm_route_override(op)


# ------------------------------------------- load policies at small shapes
#
# The non-temporal load variants (stream_loads level 1: dy and dres streamed;
# level 2: every input streamed, and the residual forward's x and r) run by
# default only at sizes where the full-size cases check them. Here every form
# is forced onto each level at small shapes, ragged and multi-block, and
# compared element by element; the route knob takes 1 + the level.

LOAD_POLICY_CASES = [
    # (form, T, heads, H, w dtype)
    ("fwd", 777, 1, 2048, "f32"),
    ("res_fwd", 333, 1, 6144, "bf16"),
    ("res_fwd", 1001, 1, 256, "f32"),
    ("bwd", 777, 1, 2048, "f32"),
    ("bwd", 3001, 1, 256, "bf16"),
    ("bwd", 129, 1, 16384, "bf16"),
    ("res_bwd", 333, 1, 6144, "bf16"),
    ("res_bwd_nodres", 333, 1, 6144, "f32"),
    ("strided_bwd", 300, 24, 256, "f32"),
]


def _check_form(form, wl, det=True):
    """Run `form` on the GPU for workload wl and check it against the oracle
    (all elements). Returns the output bits for cross-checks."""
    H, rows = wl.H, wl.rows
    w = dev_w(wl.w)
    if form in ("fwd", "res_fwd"):
        if form == "res_fwd":
            h, y, rstd = rn.rmsnorm_residual_fwd(dev_bf16(wl.x), dev_bf16(wl.r), w, wl.eps,
                                                 h=filled((rows, H)), y=filled((rows, H)))
            torch.cuda.synchronize()
            x_in = oracle.residual_add(wl.x, wl.r)
            assert np.array_equal(host_bits(h), x_in), "h not bit-exact"
        else:
            y, rstd = rn.rmsnorm_fwd(dev_bf16(wl.x), w, wl.eps, y=filled((rows, H)))
            torch.cuda.synchronize()
            x_in = wl.x
        r64, y64 = oracle.fwd(x_in, wl.w.f64, wl.eps)
        check_rstd("rstd", rstd.cpu().numpy(), r64)
        yb = host_bits(y)
        check_bf16_strict("y", yb, y64)
        return yb
    x_in = oracle.residual_add(wl.x, wl.r) if wl.r is not None else wl.x
    _, r32 = oracle_rstd32(x_in, wl.w.f64, wl.eps)
    r32_64 = r32.astype(np.float64)
    _, _, dw64 = oracle.bwd(wl.dy, x_in, r32_64, wl.w.f64, want_dx=False)
    dres = wl.dres if form == "res_bwd" else None
    if form in ("res_bwd", "res_bwd_nodres"):
        dx, dw = rn.rmsnorm_residual_bwd(dev_bf16(wl.dy), dev_bf16(x_in), dev_f32(r32), w,
                                         dres=dev_bf16(dres) if dres is not None else None,
                                         deterministic=det, dh=filled((rows, H)))
        torch.cuda.synchronize()
        dxb = host_bits(dx)
    elif form == "strided_bwd":
        row = 8192
        xbuf = dev_bf16(wl.xbuf)
        xv = xbuf[:, : wl.heads * H].unflatten(1, (wl.heads, H))
        dxbuf = filled((wl.T, row))
        dxv = dxbuf[:, : wl.heads * H].unflatten(1, (wl.heads, H))
        _, dw = rn.rmsnorm_bwd_strided(dev_bf16(wl.dy).view(wl.T, wl.heads, H), xv,
                                       dev_f32(r32).view(wl.T, wl.heads), w, deterministic=det,
                                       dx=dxv)
        torch.cuda.synchronize()
        full = host_bits(dxbuf)
        assert np.all(full[:, wl.heads * H:] == fullsize.SENTINEL), "gap columns written"
        dxb = np.ascontiguousarray(full[:, : wl.heads * H]).reshape(rows, H)
    else:
        dx, dw = rn.rmsnorm_bwd(dev_bf16(wl.dy), dev_bf16(x_in), dev_f32(r32), w,
                                deterministic=det, dx=filled((rows, H)))
        torch.cuda.synchronize()
        dxb = host_bits(dx)
    fullsize.check_dx_rows("dx", dxb, wl.dy, x_in, r32_64, wl.w.f64, dres)
    check_dw("dw", dw.cpu().numpy(), dw64)
    return dxb


@pytest.mark.parametrize("level", [0, 1, 2])
@pytest.mark.parametrize("form,T,heads,H,wdt", LOAD_POLICY_CASES)
def test_load_policy_variants(form, T, heads, H, wdt, level):
    _announce(f"load policy {form} level={level} T={T} heads={heads} H={H} w={wdt}")
    residual = form.startswith("res")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + H + level, heads=heads, residual=residual,
                    with_dres=(form != "res_bwd_nodres"),
                    strided_row=8192 if form == "strided_bwd" else 0)
    op = "fwd" if form.endswith("fwd") else "bwd"
    try:
        rn.rmsnorm_route_override(op, stream_loads=level + 1)
        got = rn.rmsnorm_route_query(op, wl.rows, H, torch.float32 if wdt == "f32" else torch.bfloat16,
                                     residual=residual)
        assert got["stream_loads"] == level
        out = _check_form(form, wl)
    finally:
        rn.rmsnorm_route_override(op)
    # the load policy changes no arithmetic: same bits as the default route
    assert np.array_equal(_check_form(form, wl), out), "load policy changed the result"


@pytest.mark.parametrize("T,heads,H,wdt,with_dres", [(300, 24, 256, "f32", True),
                                                     (50, 4, 256, "bf16", False),
                                                     (40, 2, 6144, "bf16", True)])
def test_residual_views(T, heads, H, wdt, with_dres):
    """The residual form over per-head views: x, r, h, y, dy, dres and dh each
    strided inside wider buffers whose gap columns must stay untouched;
    against the oracle, and bit-identical to the contiguous residual calls."""
    _announce(f"residual views T={T} heads={heads} H={H} w={wdt} dres={with_dres}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + heads, heads=heads, residual=True,
                    with_dres=with_dres)
    rows = wl.rows
    W = heads * H + 64  # row stride of every wide buffer

    def wide(bits, fill=None):
        buf = filled((T, W)) if fill else dev_bf16(np.zeros((T, W), np.uint16))
        if bits is not None:
            buf[:, : heads * H] = dev_bf16(bits).view(T, heads * H)
        return buf, buf[:, : heads * H].unflatten(1, (heads, H))

    w = dev_w(wl.w)
    xb, xv = wide(wl.x)
    rb, rv = wide(wl.r)
    hb, hv = wide(None, fill=True)
    yb, yv = wide(None, fill=True)
    _, _, rstd = rn.rmsnorm_residual_fwd_strided(xv, rv, w, wl.eps, h=hv, y=yv)
    torch.cuda.synchronize()
    h_ref = oracle.residual_add(wl.x, wl.r)
    for name, b in (("h", hb), ("y", yb)):
        gap = host_bits(b)[:, heads * H:]
        assert np.all(gap == fullsize.SENTINEL), f"gap columns of {name} written"
    hbits = np.ascontiguousarray(host_bits(hb)[:, : heads * H]).reshape(rows, H)
    assert np.array_equal(hbits, h_ref), "h not bit-exact"
    r64, y64 = oracle.fwd(h_ref, wl.w.f64, wl.eps)
    check_rstd("rstd", rstd.cpu().numpy().reshape(-1), r64)
    ybits = np.ascontiguousarray(host_bits(yb)[:, : heads * H]).reshape(rows, H)
    check_bf16_strict("y", ybits, y64)
    # contiguous residual forward on the same rows: same bits
    hc, yc, rc = rn.rmsnorm_residual_fwd(dev_bf16(wl.x), dev_bf16(wl.r), w, wl.eps)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(hc), hbits) and np.array_equal(host_bits(yc), ybits)
    assert torch.equal(rc, rstd.reshape(-1))
    # backward over views, fed the oracle's rstd
    r32 = oracle.round_f32(r64)
    r32_64 = r32.astype(np.float64)
    _, _, dw64 = oracle.bwd(wl.dy, h_ref, r32_64, wl.w.f64, want_dx=False)
    dyb, dyv = wide(wl.dy)
    drb, drv = wide(wl.dres) if with_dres else (None, None)
    hb2, hv2 = wide(h_ref)
    for det in (True, False):
        dhb, dhv = wide(None, fill=True)
        _, dw = rn.rmsnorm_residual_bwd_strided(dyv, hv2, dev_f32(r32).view(T, heads), w, dres=drv,
                                                deterministic=det, dh=dhv)
        torch.cuda.synchronize()
        full = host_bits(dhb)
        assert np.all(full[:, heads * H:] == fullsize.SENTINEL), "gap columns of dh written"
        dhbits = np.ascontiguousarray(full[:, : heads * H]).reshape(rows, H)
        fullsize.check_dx_rows(f"dh det={det}", dhbits, wl.dy, h_ref, r32_64, wl.w.f64,
                               wl.dres if with_dres else None)
        check_dw(f"dw det={det}", dw.cpu().numpy(), dw64)
        dhc, dwc = rn.rmsnorm_residual_bwd(dev_bf16(wl.dy), dev_bf16(h_ref), dev_f32(r32), w,
                                           dres=dev_bf16(wl.dres) if with_dres else None,
                                           deterministic=det)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(dhc), dhbits), "views changed dh"
        if det:
            assert torch.equal(dwc.view(torch.int32), dw.view(torch.int32)), "views changed dw"


# ------------------------------------------------------ non-finite inputs

@pytest.mark.parametrize("nan_in_x", [False, True])
@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("T", [48, 300])
def test_non_finite_inputs_propagate_like_the_oracle(T, wdt, nan_in_x):
    """Nothing special-cases non-finite inputs: +inf in x, NaN in dy (and
    NaN in x) leave NaN exactly where the FP64 oracle has NaN in y, rstd, dx
    and dw (row 9 with +inf gets rstd 0), and every other element stays
    within the usual budgets. T 48 takes the column-task kernel, T 300 the
    row kernel."""
    H = 1024
    _announce(f"non-finite T={T} H={H} w={wdt} nan_in_x={nan_in_x}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=11 + T)
    x, dy = wl.x.copy(), wl.dy.copy()
    x[9, 3] = 0x7F80       # +inf
    dy[20, 100] = 0x7FC0   # NaN
    if nan_in_x:
        x[5, 17] = 0x7FC0
    r64, y64 = oracle.fwd(x, wl.w.f64, wl.eps)
    r32 = oracle.round_f32(r64)
    dx64, c64, dw64 = oracle.bwd(dy, x, r32.astype(np.float64), wl.w.f64)
    w = dev_w(wl.w)
    y, rstd = rn.rmsnorm_fwd(dev_bf16(x), w, wl.eps)
    dx, dw = rn.rmsnorm_bwd(dev_bf16(dy), dev_bf16(x), dev_f32(r32), w, deterministic=True)
    dx_nd, dw_nd = rn.rmsnorm_bwd(dev_bf16(dy), dev_bf16(x), dev_f32(r32), w, deterministic=False)
    torch.cuda.synchronize()
    yb, rs, dxb, dwn = host_bits(y), rstd.cpu().numpy(), host_bits(dx), dw.cpu().numpy()
    assert np.array_equal(np.isnan(to_f64(yb)), np.isnan(y64)), "y NaN pattern"
    assert np.array_equal(np.isnan(rs), np.isnan(r64)), "rstd NaN pattern"
    assert rs[9] == 0.0 and r64[9] == 0.0
    assert np.array_equal(np.isnan(to_f64(dxb)), np.isnan(dx64)), "dx NaN pattern"
    assert np.array_equal(np.isnan(dwn), np.isnan(dw64)), "dw NaN pattern"
    assert np.array_equal(host_bits(dx_nd), dxb), "dx differs between modes"
    assert np.array_equal(np.isnan(dw_nd.cpu().numpy()), np.isnan(dw64)), "non-det dw NaN pattern"
    fy = ~np.isnan(y64)
    check_bf16_strict("y (finite)", yb[fy], y64[fy])
    fr = np.isfinite(r64) & (r64 != 0.0)
    check_rstd("rstd (finite)", rs[fr], r64[fr])
    rows = np.isfinite(dx64).all(axis=1)
    E = dx_bound(to_f64(x[rows]), to_f64(dy[rows]), wl.w.f64, r32.astype(np.float64)[rows],
                 c64[rows], H)
    check_dx("dx (finite rows)", dxb[rows], dx64[rows], E)
    fc = ~np.isnan(dw64)
    check_dw("dw (finite columns)", dwn[fc], dw64[fc])
    assert nan_in_x == bool(np.isnan(dw64).all())
