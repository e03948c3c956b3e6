"""The checkpointed training step and the backward that recomputes rstd.

The pages time a third op beside fwd and bwd: "2xfwd+bwd", the checkpointed
step of forward, forward recompute, backward (flashinfer PR
"fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy backward routes", "Key").
rmsnorm_bwd_recompute folds the recompute into the backward: it takes no
rstd and forms each row's rstd from x with the forward's arithmetic.

Checks:
* against the oracle at its own rstd (FP64, rounded to FP32): dw within the
  budget for both rstd forms; dx within one BF16 ulp of RNE(dx64), or, where
  the FP32 evaluation bound says so, within ulp + E_rc. E_rc adds to the
  bound E of the plain backward the effect of the kernel's rstd differing
  from the oracle's by up to one FP32 ulp: d(dx)/d(rstd) = g - 3 xhat c, so
  |delta dx| <= 2^-23 rstd (|g| + 3 |xhat c|).
* bit for bit against the plain backward fed the GPU forward's rstd, where
  both run the row kernel (rows > 64) and the plain backward is forced
  (route override) onto the recompute route's launch shape and partition:
  the recomputed rstd equals the forward's (the FP64 sum of the FP32 group
  sums is exact for these inputs). The two routes' default shapes differ
  (the recompute form has its own table), and with them the summation
  order of the row dot products and of dw.
* the checkpointed step as one HIP graph, replayed several times with eager
  work in between: every replay reproduces the eager result bit for bit, and
  the recompute forward reproduces the first forward's y and rstd.
"""
from __future__ import annotations

import contextlib

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import synth
from tests.parity import check_dw, check_dx, dx_bound, oracle_rstd32, to_f64
from tests.test_parity_gpu import DEV, _announce, dev_bf16, dev_f32, dev_w, host_bits

pytestmark = pytest.mark.gpu


# CUs the row kernels' fixed partition is sized for (grid = min(tiles, 256 x
# blocks per CU))
PARTITION_CUS = 256


@contextlib.contextmanager
def recompute_shape(rows, H, w_dtype):
    """Run the plain backward at the launch shape the recompute form routes
    to, so that both sum in the same order."""
    r = rn.rmsnorm_route_query("bwd", rows, H, w_dtype, recompute=True)
    rn.rmsnorm_route_override("bwd", vec_per_lane=r["vec_per_lane"], unroll=r["unroll"],
                              rows_per_block=r["rows_per_block"],
                              blocks_per_cu=-(-r["grid"] // PARTITION_CUS))
    try:
        p = rn.rmsnorm_route_query("bwd", rows, H, w_dtype)
        assert (p["vec_per_lane"], p["unroll"], p["rows_per_block"], p["grid"]) == \
            (r["vec_per_lane"], r["unroll"], r["rows_per_block"], r["grid"])
        yield
    finally:
        rn.rmsnorm_route_override("bwd")


def _rc_bound(wl, r32, c64):
    """E_rc - E: the dx change from a one-ulp FP32 difference in rstd."""
    x64, dy64 = to_f64(wl.x), to_f64(wl.dy)
    rs = r32.astype(np.float64)[:, None]
    g = dy64 * wl.w.f64[None, :]
    xhat = x64 * rs
    return 2.0 ** -23 * rs * (np.abs(g) + 3.0 * np.abs(xhat * c64[:, None]))


SMALL_RC = [
    (1, 8, "f32"), (3, 24, "bf16"), (64, 256, "f32"), (65, 4096, "bf16"), (300, 2048, "f32"),
    (129, 6144, "bf16"), (257, 16384, "bf16"), (1000, 512, "f32"), (9000, 128, "bf16"),
    (700, 5120, "f32"), (2049, 1536, "bf16"), (70, 1032, "bf16"),
]


@pytest.mark.parametrize("T,H,wdt", SMALL_RC)
def test_bwd_recompute_small(T, H, wdt):
    _announce(f"bwd_recompute T={T} H={H} w={wdt}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=5 * T + H)
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64)
    _, _, dw64_i = oracle.bwd(wl.dy, wl.x, r64, wl.w.f64, want_dx=False)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32.astype(np.float64), c64, H)
    E = E + _rc_bound(wl, r32, c64)
    x, dy, w = dev_bf16(wl.x), dev_bf16(wl.dy), dev_w(wl.w)
    outs = {}
    for det in (True, False):
        dx, dw = rn.rmsnorm_bwd_recompute(dy, x, w, wl.eps, deterministic=det)
        torch.cuda.synchronize()
        outs[det] = (host_bits(dx), dw.cpu().numpy())
        check_dx(f"dx det={det}", outs[det][0], dx64, E)
        check_dw(f"dw det={det} (forward's rstd)", outs[det][1], dw64)
        check_dw(f"dw det={det} (FP64 rstd)", outs[det][1], dw64_i)
    assert np.array_equal(outs[True][0], outs[False][0]), "dx differs between modes"
    for _ in range(3):
        dx2, dw2 = rn.rmsnorm_bwd_recompute(dy, x, w, wl.eps, deterministic=True)
        torch.cuda.synchronize()
        assert np.array_equal(dw2.cpu().numpy().view(np.uint32), outs[True][1].view(np.uint32))
        assert np.array_equal(host_bits(dx2), outs[True][0])
    if T > 64:
        _, rstd = rn.rmsnorm_fwd(x, w, wl.eps)
        with recompute_shape(T, H, w.dtype):
            dxp, dwp = rn.rmsnorm_bwd(dy, x, rstd, w, deterministic=True)
            torch.cuda.synchronize()
        assert np.array_equal(host_bits(dxp), outs[True][0]), "dx differs from the plain backward"
        assert np.array_equal(dwp.cpu().numpy().view(np.uint32), outs[True][1].view(np.uint32)), \
            "dw differs from the plain backward"


@pytest.mark.parametrize("T,heads,H,row", [(300, 24, 256, 8192), (50, 4, 256, 1024), (7, 3, 512, 2048)])
def test_bwd_recompute_strided_heads(T, heads, H, row):
    _announce(f"bwd_recompute strided T={T} heads={heads} H={H} row={row}")
    wl = synth.make(T=T, H=H, w_dtype="f32", seed=T + heads + 11, heads=heads, strided_row=row)
    xbuf = dev_bf16(wl.xbuf)
    xview = xbuf[:, : heads * H].unflatten(1, (heads, H))
    w = dev_w(wl.w)
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32.astype(np.float64), c64, H)
    E = E + _rc_bound(wl, r32, c64)
    dy = dev_bf16(wl.dy).view(T, heads, H)
    sentinel = 0x7FC0
    dxbuf = torch.full((T, row), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    dxview = dxbuf[:, : heads * H].unflatten(1, (heads, H))
    _, dw = rn.rmsnorm_bwd_recompute(dy, xview, w, wl.eps, deterministic=True, dx=dxview)
    torch.cuda.synchronize()
    full = host_bits(dxbuf)
    assert np.all(full[:, heads * H:] == sentinel), "gap columns of the dx buffer were written"
    dx_rc = np.ascontiguousarray(full[:, : heads * H]).reshape(-1, H)
    check_dx("dx", dx_rc, dx64, E)
    check_dw("dw", dw.cpu().numpy(), dw64)
    if T * heads > 64:
        _, rstd = rn.rmsnorm_fwd_strided(xview, w, wl.eps)
        with recompute_shape(T * heads, H, w.dtype):
            dxp, dwp = rn.rmsnorm_bwd_strided(dy, xview, rstd, w, deterministic=True)
            torch.cuda.synchronize()
        assert np.array_equal(host_bits(dxp).reshape(-1, H), dx_rc)
        assert torch.equal(dwp.view(torch.int32), dw.view(torch.int32))


FULL = ["c2_T4096_H4096_bf16w", "c3_T131072_H2048_f32w_heavy",
        "c5a_heads_T32768x24x256_strided8192_f32w", "c5b_heads_T32768x4x256_f32w"]


@pytest.mark.parametrize("name", FULL)
def test_bwd_recompute_full_size(name):
    """At the full workload sizes: bit-identical to the plain backward fed
    the GPU forward's rstd at the same launch shape (every row and column),
    and dw against the oracle."""
    _announce(f"bwd_recompute full {name}")
    wl = synth.config(name, seed=0)
    w = dev_w(wl.w)
    with recompute_shape(wl.rows, wl.H, w.dtype):
        x, dy, dxp, dwp = _plain_full(wl, w)
    for det in (True, False):
        dx, dw = rn.rmsnorm_bwd_recompute(dy, x, w, wl.eps, deterministic=det)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), dxp.view(torch.int16)), f"dx det={det}"
        assert torch.equal(dw.view(torch.int32), dwp.view(torch.int32)), f"dw det={det}"
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    _, _, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64, want_dx=False)
    _, _, dw64_i = oracle.bwd(wl.dy, wl.x, r64, wl.w.f64, want_dx=False)
    worst = check_dw("dw (forward's rstd)", dw.cpu().numpy(), dw64)
    worst_i = check_dw("dw (FP64 rstd)", dw.cpu().numpy(), dw64_i)
    print(f"{name}: recompute dw worst {worst:.2e} / {worst_i:.2e} of budget", flush=True)


def _plain_full(wl, w):
    """GPU forward, then the plain deterministic backward fed its rstd."""
    if wl.xbuf is not None:
        T, heads, H = wl.T, wl.heads, wl.H
        xbuf = dev_bf16(wl.xbuf)
        x = xbuf[:, : heads * H].unflatten(1, (heads, H))
        dy = dev_bf16(wl.dy).view(T, heads, H)
        _, rstd = rn.rmsnorm_fwd_strided(x, w, wl.eps)
        dxp, dwp = rn.rmsnorm_bwd_strided(dy, x, rstd, w, deterministic=True)
    else:
        x = dev_bf16(wl.x)
        dy = dev_bf16(wl.dy)
        if wl.heads > 1:
            x = x.view(wl.T, wl.heads, wl.H)
            dy = dy.view(wl.T, wl.heads, wl.H)
            _, rstd = rn.rmsnorm_fwd_strided(x, w, wl.eps)
            dxp, dwp = rn.rmsnorm_bwd_strided(dy, x, rstd, w, deterministic=True)
        else:
            _, rstd = rn.rmsnorm_fwd(x, w, wl.eps)
            dxp, dwp = rn.rmsnorm_bwd(dy, x, rstd, w, deterministic=True)
    torch.cuda.synchronize()
    return x, dy, dxp, dwp


@pytest.mark.parametrize("recompute_in_bwd", [False, True])
@pytest.mark.parametrize("T,H,wdt", [(4096, 4096, "bf16"), (333, 2048, "f32")])
def test_checkpointed_step_graph(T, H, wdt, recompute_in_bwd):
    """forward, forward recompute, backward (or forward, recompute backward)
    captured in one HIP graph and replayed several times."""
    _announce(f"checkpointed step T={T} H={H} w={wdt} recompute_in_bwd={recompute_in_bwd}")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + 2 * H)
    x, dy, w = dev_bf16(wl.x), dev_bf16(wl.dy), dev_w(wl.w)
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(x)
    rs1 = torch.empty(T, dtype=torch.float32, device=DEV)
    rs2 = torch.empty_like(rs1)
    dx = torch.empty_like(x)
    dw = torch.empty(H, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(rn.rmsnorm_bwd_workspace_bytes(T, H, w.dtype, True), 256) + 256,
                     dtype=torch.uint8, device=DEV)
    ws = ws[(-ws.data_ptr()) % 256:]

    def step():
        rn.rmsnorm_fwd(x, w, wl.eps, y=y1, rstd=rs1)
        if recompute_in_bwd:
            rn.rmsnorm_bwd_recompute(dy, x, w, wl.eps, deterministic=True, dx=dx, dw=dw, workspace=ws)
        else:
            rn.rmsnorm_fwd(x, w, wl.eps, y=y2, rstd=rs2)
            rn.rmsnorm_bwd(dy, x, rs2, w, deterministic=True, dx=dx, dw=dw, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in (("y1", y1), ("rs1", rs1), ("dx", dx), ("dw", dw))}
    if not recompute_in_bwd:
        assert torch.equal(y2.view(torch.int16), y1.view(torch.int16)), "recompute changed y"
        assert torch.equal(rs2, rs1), "recompute changed rstd"
    r64, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    dx64, c64, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64)
    E = dx_bound(to_f64(wl.x), to_f64(wl.dy), wl.w.f64, r32.astype(np.float64), c64, H)
    check_dx("dx", host_bits(dx), dx64, E + _rc_bound(wl, r32, c64) if recompute_in_bwd else E)
    check_dw("dw", dw.cpu().numpy(), dw64)

    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(device=DEV)
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            step()
    torch.cuda.synchronize()
    for i in range(3):
        for t in (y1, rs1, dx, dw):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), ref["y1"].view(torch.int16)), f"replay {i}: y"
        assert torch.equal(rs1, ref["rs1"]), f"replay {i}: rstd"
        assert torch.equal(dx.view(torch.int16), ref["dx"].view(torch.int16)), f"replay {i}: dx"
        assert torch.equal(dw.view(torch.int32), ref["dw"].view(torch.int32)), f"replay {i}: dw"
        # eager work between replays
        step()
        torch.cuda.synchronize()
