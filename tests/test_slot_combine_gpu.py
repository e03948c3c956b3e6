"""The backward row kernel's two ways of combining its row slots' dw sums.

A block of the row kernel holds rows_per_block row slots, each with its own
FP64 dw sums per column; before the block writes its partial row the slots
are added in slot order. From four slots up, when [slots, H] doubles fit in
64 KB of LDS, every slot stores its sums at once and each thread folds whole
column pairs (the one-step kernels); otherwise the slots are added one per
round through an [H] area (the serial kernels). Both add in the same order.

The cases below hit each kernel family on purpose (the test asserts which one
the route takes): FP32 and FP64 partial rows, rows of one wave and of
several, slot counts of 4, 6, 8, 16 and 32 (6 leaves a remainder after
the fold's groups of four; 4 at H 2560 is over the LDS limit, so serial),
the plain, residual (with and without dres), per-head strided and
recompute forms. Every element of dx (dh) is held to the oracle's bound and
dw to its budget; deterministic dw is checked bit for bit over repeated
calls; the recompute form is checked against the plain backward run at its
launch shape (same summation order) fed the GPU forward's rstd.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import synth
from tests.parity import check_dw, oracle_rstd32
from tests.test_parity_gpu import DEV, _announce, _bwd_case, _check_form, dev_bf16, dev_w
from tests.test_recompute_gpu import recompute_shape

pytestmark = pytest.mark.gpu

COMB_ALL_LDS = 64 * 1024     # bytes of slot sums the one-step kernels hold
F32_PARTIAL_MAX_ROWS = 8192  # FP32 partial rows up to this many rows, FP64 above

# (form, T, heads, H, w dtype, route override or None, one-step combine expected)
CASES = [
    ("bwd", 9000, 1, 256, "f32", None, True),                 # 16 slots, FP64 partials
    ("bwd", 4096, 1, 256, "bf16", None, True),                # 16 slots, FP32
    ("bwd", 5000, 1, 1024, "f32", None, True),                # 6 slots of 128 lanes
    ("bwd", 9001, 1, 1536, "bf16", None, True),               # 4 slots of 192 lanes, FP64
    ("bwd", 3000, 1, 2048, "f32", None, True),                # 4 x 2048 doubles: the limit
    ("bwd", 2000, 1, 256, "f32", dict(vec_per_lane=4, rows_per_block=32), True),
    ("bwd", 2000, 1, 2560, "bf16", dict(vec_per_lane=4, rows_per_block=4), False),
    ("bwd", 3000, 1, 4096, "bf16", None, False),              # 2 slots: serial
    ("res_bwd", 3000, 1, 512, "bf16", None, True),            # 8 slots, 2 rows per iteration
    ("res_bwd_nodres", 9000, 1, 256, "f32", None, True),
    ("strided_bwd", 300, 24, 256, "f32", None, True),
    ("rc_bwd", 9000, 1, 256, "f32", None, True),
    ("rc_bwd", 3000, 1, 512, "bf16", None, True),             # recompute table: 4 slots
    ("rc_bwd", 3000, 1, 1024, "bf16", None, False),           # recompute table: 2 slots
]


def _wdt(w):
    return torch.float32 if w == "f32" else torch.bfloat16


@pytest.mark.parametrize("form,T,heads,H,wdt,knobs,one_step", CASES)
def test_slot_combine(form, T, heads, H, wdt, knobs, one_step):
    _announce(f"slot combine {form} T={T} heads={heads} H={H} w={wdt} {knobs}")
    residual = form.startswith("res")
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + 7 * H + heads, heads=heads, residual=residual,
                    with_dres=(form == "res_bwd"), strided_row=8192 if form == "strided_bwd" else 0)
    rows = wl.rows
    if knobs:
        rn.rmsnorm_route_override("bwd", **knobs)
    try:
        r = rn.rmsnorm_route_query("bwd", rows, H, _wdt(wdt), residual=residual,
                                   recompute=(form == "rc_bwd"))
        rpb = r["rows_per_block"]
        assert (rpb >= 4 and rpb * H * 8 <= COMB_ALL_LDS) == one_step, r
        assert r["partial_f64"] == (1 if rows > F32_PARTIAL_MAX_ROWS else 0), r
        if form == "rc_bwd":
            _check_recompute(wl)
        else:
            _check_form(form, wl)
            if form == "bwd":
                _, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
                dws = [_bwd_case(wl, True, r32)[1] for _ in range(3)]
                for dw in dws[1:]:
                    assert np.array_equal(dw.view(np.uint32), dws[0].view(np.uint32)), \
                        "deterministic dw changed between calls"
    finally:
        rn.rmsnorm_route_override("bwd")


def _check_recompute(wl):
    H, rows = wl.H, wl.rows
    x, dy, w = dev_bf16(wl.x), dev_bf16(wl.dy), dev_w(wl.w)
    _, rstd = rn.rmsnorm_fwd(x, w, wl.eps)
    dx_rc, dw_rc = rn.rmsnorm_bwd_recompute(dy, x, w, wl.eps)
    torch.cuda.synchronize()
    # dw within the budget against the oracle at its own rstd rounded to FP32
    _, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    _, _, dw64 = oracle.bwd(wl.dy, wl.x, r32.astype(np.float64), wl.w.f64, want_dx=False)
    check_dw("dw (recompute)", dw_rc.cpu().numpy(), dw64)
    # the plain backward at the recompute route's launch shape, fed the
    # forward's rstd, sums in the same order: same bits
    with recompute_shape(rows, H, w.dtype):
        dx_p, dw_p = rn.rmsnorm_bwd(dy, x, rstd, w, deterministic=True)
        torch.cuda.synchronize()
    assert torch.equal(dx_rc.view(torch.int16), dx_p.view(torch.int16)), "dx differs from plain"
    assert torch.equal(dw_rc.view(torch.int32), dw_p.view(torch.int32)), "dw differs from plain"
