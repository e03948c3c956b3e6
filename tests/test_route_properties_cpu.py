"""Properties of the route table over 4000 seeded random shapes (no GPU).

The kernels assume things about the launch shapes the route table hands
them: a row group's lanes cover the row, a block holds its row groups, the
grid fits the fixed partition, the workspace query covers the partial rows
the backward writes, the allocation-free entry point's fixed scratch holds
every default route's partials, and the deterministic partition depends on
the shape only (not on the weight dtype, the mode or the form). These are
checked here for every operation and form, with token counts log-uniform up
to the 2^31 - 1 row limit and every multiple of 8 up to 16384 as the width.
"""
import ctypes
import math

import numpy as np

from bwd_rmsnorm_fwd_02_amd import _lib

lib = _lib.load()

OP_FWD, OP_BWD, OP_LN_FWD, OP_LN_BWD = 0, 1, 2, 3
FORM_PLAIN, FORM_RESIDUAL, FORM_RECOMPUTE = 0, 1, 2
ROW_LIMIT = 2 ** 31 - 1
NOALLOC_SCRATCH = 32 << 20     # the allocation-free entry point's fixed array
PARTITION_CUS = 256


def route(op, rows, H, wdt, det, form):
    info = _lib.RouteInfo()
    st = lib.rmsnorm_route_query(op, rows, H, wdt, det, form, ctypes.byref(info))
    return st, info


def _shapes(n=4000, seed=20261203):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        rows = int(round(math.exp(rng.uniform(0.0, math.log(ROW_LIMIT)))))
        rows = max(1, min(rows, ROW_LIMIT))
        H = 8 * int(rng.integers(1, 2049))
        yield rows, H, int(rng.integers(2))


def _check_row_layout(r, H, where):
    nvec = H // 8
    assert r.vec_per_lane in (1, 2, 4), where
    assert r.unroll in (1, 2, 4, 8), where
    assert r.vec_per_lane * r.lanes_per_row >= nvec, where
    lpr = r.lanes_per_row
    assert (lpr <= 64 and lpr & (lpr - 1) == 0) or lpr % 64 == 0, where
    assert r.block_threads == lpr * r.rows_per_block <= 1024, where
    assert 1 <= r.grid <= PARTITION_CUS * 32, where
    assert r.stream_loads in (0, 1, 2), where


def test_route_properties_over_random_shapes():
    for rows, H, wdt in _shapes():
        for form in (FORM_PLAIN, FORM_RESIDUAL):
            st, f = route(OP_FWD, rows, H, wdt, 1, form)
            where = ("fwd", rows, H, wdt, form)
            assert st == 0, where
            assert f.kind == _lib.RMSN_KIND_FWD_ROW, where
            _check_row_layout(f, H, where)
            # no idle block: the last block's first tile starts below rows
            assert (f.grid - 1) * f.rows_per_block * f.unroll < rows, where

        ws = {det: lib.rmsnorm_bwd_workspace_bytes(rows, H, wdt, det) for det in (0, 1)}
        ref = None
        for form in (FORM_PLAIN, FORM_RESIDUAL, FORM_RECOMPUTE):
            for det in (0, 1):
                st, b = route(OP_BWD, rows, H, wdt, det, form)
                where = ("bwd", rows, H, wdt, det, form)
                assert st == 0, where
                if rows <= 64 and form != FORM_RECOMPUTE:
                    assert b.kind == _lib.RMSN_KIND_BWD_COLTASK, where
                    continue
                # both modes take the fixed-order two-stage path by default
                assert b.kind == _lib.RMSN_KIND_BWD_ROW_DET, where
                _check_row_layout(b, H, where)
                assert b.partials == b.grid, where
                assert b.partial_f64 == (1 if rows > 8192 else 0), where
                assert (b.grid - 1) * b.rows_per_block * b.unroll < rows, where
                part = b.partials * H * (8 if b.partial_f64 else 4)
                assert ws[det] >= part, where
                # the reduce's column blocks cover the row
                assert b.reduce_grid * 16 * (2 if b.partial_f64 else 4) >= H, where
                if form == FORM_PLAIN:
                    # the fixed scratch of the allocation-free entry point
                    assert part <= NOALLOC_SCRATCH, where
                if form != FORM_RECOMPUTE:
                    shape = (b.grid, b.rows_per_block, b.unroll, b.vec_per_lane, b.lanes_per_row,
                             b.partial_f64)
                    # the partition is a function of (rows, H) alone
                    if ref is None:
                        ref = shape
                    assert shape == ref, where
                    for w2 in (0, 1):
                        assert route(OP_BWD, rows, H, w2, det, form)[1].grid == b.grid, where


def test_layernorm_route_properties_over_random_shapes():
    for rows, H, wdt in _shapes(n=2000, seed=7):
        st, f = route(OP_LN_FWD, rows, H, wdt, 1, FORM_PLAIN)
        assert st == 0
        _check_row_layout(f, H, ("ln_fwd", rows, H))
        assert (f.grid - 1) * f.rows_per_block * f.unroll < rows
        for det in (0, 1):
            st, b = route(OP_LN_BWD, rows, H, wdt, det, FORM_PLAIN)
            where = ("ln_bwd", rows, H, wdt, det)
            assert st == 0, where
            _check_row_layout(b, H, where)
            assert b.partials == b.grid, where
            need = lib.layernorm_bwd_workspace_bytes(rows, H, wdt, det)
            # dgamma and dbeta partial rows, [P, 2H]
            assert need >= b.partials * 2 * H * (8 if b.partial_f64 else 4), where
