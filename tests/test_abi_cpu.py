"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, validates arguments before enqueueing anything, and its route table
(the analogue of the pages' registry-window test, which also runs without a
GPU) picks the documented kernels.

Calls that would pass validation are never made here: every call below
returns an error code from the host checks, so fake (never dereferenced)
pointers are safe. On a machine with a GPU the fake-pointer cases are
skipped all the same.
"""
import ctypes
import os
import re

import pytest

from bwd_rmsnorm_fwd_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm.h")

lib = _lib.load()
P = ctypes.c_void_p


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b((?:rmsnorm|layernorm)_\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declarations_are_exported():
    names = _declared_functions()
    assert len(names) >= 12
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(-10, 1):
        s = _lib.status_string(code)
        assert s and s != "unknown status", code
    assert _lib.status_string(-100) == "unknown status"


def _fake(addr):
    return P(addr)


import torch  # noqa: E402

_gpu_visible = torch.cuda.device_count() > 0
fake_only = pytest.mark.skipif(_gpu_visible, reason="fake-pointer cases run only without a GPU")


@fake_only
def test_fwd_argument_errors():
    A = 0x100000
    s = P(0)
    f = lib.rmsnorm_fwd
    assert f(_fake(A), _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), 4, 7, s) == -3
    assert f(_fake(A), _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), 4, 16392, s) == -3
    assert f(_fake(A), _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), -1, 64, s) == -3
    assert f(_fake(A), _fake(A + 0x100000), 5, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), 4, 64, s) == -2
    assert f(None, _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), 4, 64, s) == -1
    assert f(_fake(A + 2), _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 0x300000), 4, 64, s) == -4
    assert f(_fake(A), _fake(A + 0x100000), 0, -1.0, _fake(A + 0x200000), _fake(A + 0x300000), 4, 64, s) == -9
    assert f(_fake(A), _fake(A + 0x100000), 0, float("nan"), _fake(A + 0x200000), _fake(A + 0x300000), 4, 64, s) == -9
    # y overlapping x but not exactly in place
    assert f(_fake(A), _fake(A + 0x100000), 0, 1e-6, _fake(A + 64), _fake(A + 0x300000), 4, 64, s) == -7
    # rstd inside x
    assert f(_fake(A), _fake(A + 0x100000), 0, 1e-6, _fake(A + 0x200000), _fake(A + 16), 4, 64, s) == -7
    # zero rows: no-op, no launch
    assert f(None, None, 0, 1e-6, None, None, 0, 64, s) == 0


@fake_only
def test_strided_view_errors():
    A = 0x1000000
    s = P(0)
    V = _lib.View
    f = lib.rmsnorm_fwd_strided
    xv = V(10, 24, 256, 8192, 256)
    yv = V(10, 24, 256, 24 * 256, 256)
    W, Y, R = A + 0x1000000, A + 0x2000000, A + 0x3000000
    # stride not a multiple of 8 elements
    assert f(_fake(A), V(10, 24, 256, 8190, 256), _fake(W), 1, 1e-6, _fake(Y), yv, _fake(R), s) == -4
    # views disagree on heads
    assert f(_fake(A), xv, _fake(W), 1, 1e-6, _fake(Y), V(10, 23, 256, 24 * 256, 256), _fake(R), s) == -3
    # output rows overlapping each other
    assert f(_fake(A), xv, _fake(W), 1, 1e-6, _fake(Y), V(10, 24, 256, 24 * 256, 128), _fake(R), s) == -7
    # negative stride
    assert f(_fake(A), V(10, 24, 256, -8192, 256), _fake(W), 1, 1e-6, _fake(Y), yv, _fake(R), s) == -3
    # offset overflow
    assert f(_fake(A), V(10, 24, 256, 1 << 62, 256), _fake(W), 1, 1e-6, _fake(Y), yv, _fake(R), s) == -6


@fake_only
def test_bwd_argument_errors():
    A = 0x4000000
    s = P(0)
    f = lib.rmsnorm_bwd
    T, H = 4096, 4096
    DY, X, RS, W, DX, DW, WS = (A + i * 0x4000000 for i in range(7))
    need = lib.rmsnorm_bwd_workspace_bytes(T, H, 0, 1)
    assert need > 0
    # the query covers every backward form; the plain route's own partial
    # rows need this much
    st, r = route(1, T, H, 0, 1, 0)
    assert st == 0 and r.partials > 0
    plain = -(-r.partials * H * (8 if r.partial_f64 else 4) // 256) * 256
    assert need >= plain
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), _fake(DW), T, H, _fake(WS), plain - 1, s) == -5
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), _fake(DW), T, H, None, need, s) == -5
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), _fake(DW), T, H, _fake(WS + 8), need, s) == -5
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), None, T, H, _fake(WS), need, s) == -1
    # dx in place over dy is not allowed in the backward
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DY), _fake(DW), T, H, _fake(WS), need, s) == -7
    # workspace overlapping dx
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), _fake(DW), T, H, _fake(DX), need, s) == -7
    # dw inside x
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W), 0, 1, _fake(DX), _fake(X + 64), T, H, _fake(WS), need, s) == -7
    # misaligned FP32 weight
    assert f(_fake(DY), _fake(X), _fake(RS), _fake(W + 4), 1, 1, _fake(DX), _fake(DW), T, H, _fake(WS), need, s) == -4


@fake_only
def test_bwd_recompute_argument_errors():
    A = 0x40000000
    s = P(0)
    V = _lib.View
    f = lib.rmsnorm_bwd_recompute
    T, H = 4096, 2048
    v = V(T, 1, H, H, 0)
    DY, X, W, DX, DW, WS = (A + i * 0x4000000 for i in range(6))
    need = lib.rmsnorm_bwd_workspace_bytes(T, H, 1, 1)
    args = lambda **k: [_fake(k.get("dy", DY)), v, _fake(k.get("x", X)) if k.get("x", X) else None, v,
                        _fake(W), 1, k.get("eps", 1e-6), 1, _fake(k.get("dx", DX)), v, _fake(DW),
                        _fake(WS), k.get("ws", need), s]
    assert f(*args(eps=-1.0)) == -9
    assert f(*args(eps=float("nan"))) == -9
    assert f(*args(eps=float("inf"))) == -9
    assert f(*args(x=0)) == -1
    assert f(*args(dx=X)) == -7          # dx over x
    assert f(*args(ws=need - 1)) == -5
    # views must agree
    assert f(_fake(DY), v, _fake(X), V(T, 1, H + 8, H + 8, 0), _fake(W), 1, 1e-6, 1, _fake(DX), v,
             _fake(DW), _fake(WS), need, s) == -3


@fake_only
def test_residual_view_argument_errors():
    A = 0x80000000
    s = P(0)
    V = _lib.View
    T, heads, H = 64, 4, 256
    c = V(T, heads, H, heads * H, H)
    X, R, W, Hh, Y, RS = (A + i * 0x1000000 for i in range(6))
    f = lib.rmsnorm_residual_fwd_strided
    ok = lambda **k: [_fake(X), k.get("xv", c), _fake(k.get("r", R)) if k.get("r", R) else None,
                      k.get("rv", c), _fake(W), 1, 1e-6, _fake(k.get("h", Hh)), k.get("hv", c),
                      _fake(k.get("y", Y)), k.get("yv", c), _fake(RS), s]
    assert f(*ok(r=0)) == -1
    assert f(*ok(rv=V(T, heads + 1, H, heads * H, H))) == -3     # views disagree
    assert f(*ok(hv=V(T, heads, H, -heads * H, H))) == -3        # negative stride
    assert f(*ok(rv=V(T, heads, H, heads * H + 4, H))) == -4     # stride not 16-byte aligned
    assert f(*ok(h=R)) == -7                                     # h over r
    assert f(*ok(y=X + 16)) == -7                                # y overlapping x
    assert f(*ok(hv=V(T, heads, H, heads * H, H // 2))) == -7    # h rows overlap each other
    assert f(None, V(0, heads, H, heads * H, H), None, V(0, heads, H, heads * H, H), None, 1, 1e-6,
             None, V(0, heads, H, heads * H, H), None, V(0, heads, H, heads * H, H), None, s) == 0
    g = lib.rmsnorm_residual_bwd_strided
    DY, HH, DR, RS2, W2, DH, DW, WS = (A + 0x8000000 + i * 0x1000000 for i in range(8))
    need = lib.rmsnorm_bwd_workspace_bytes(T * heads, H, 1, 1)
    bad = V(T, heads, H, heads * H + 8, H)
    args = lambda **k: [_fake(DY), c, _fake(HH), c, _fake(k.get("dr", DR)) if k.get("dr", DR) else None,
                        k.get("drv", c), _fake(RS2), _fake(W2), 1, 1, _fake(k.get("dh", DH)), c,
                        _fake(DW), _fake(WS), need, s]
    assert g(*args(drv=V(T, heads, H + 8, heads * H, H))) == -3  # dres view disagrees
    assert g(*args(drv=V(T, heads, H, -8, H))) == -3             # negative stride
    assert g(*args(dh=DR)) == -7                                 # dh over dres
    assert g(*args(dh=HH)) == -7                                 # dh over h
    # a NULL dres ignores its view
    assert g(*args(dr=0, drv=bad, dh=HH)) == -7


# ------------------------------------------------------------------ routes

def route(op, rows, H, wdt=0, det=1, res=0):
    info = _lib.RouteInfo()
    st = lib.rmsnorm_route_query(op, rows, H, wdt, det, res, ctypes.byref(info))
    return st, info


def test_route_small_t_uses_column_tasks_in_both_modes():
    for det in (0, 1):
        for rows in (1, 2, 63, 64):
            st, r = route(1, rows, 256, 1, det)
            assert st == 0 and r.kind == _lib.RMSN_KIND_BWD_COLTASK
        st, r = route(1, 65, 256, 1, det)
        # above the column-task window both modes run the two-stage path by
        # default (the atomic finalise measured slower on MI355X)
        assert r.kind == _lib.RMSN_KIND_BWD_ROW_DET


def test_route_recompute_form_runs_the_row_kernel_at_every_t():
    for det in (0, 1):
        for rows in (1, 2, 64, 65, 4096, 131072):
            st, r = route(1, rows, 256, 1, det, 2)
            assert st == 0 and r.kind == _lib.RMSN_KIND_BWD_ROW_DET
            _, plain = route(1, rows, 256, 1, det, 0)
            if rows > 64:
                # at H 256 the recompute table takes the plain backward's shape
                for f in ("grid", "vec_per_lane", "lanes_per_row", "rows_per_block", "unroll",
                          "partials", "partial_f64"):
                    assert getattr(r, f) == getattr(plain, f), f
    # the workspace query covers the recompute form's partials at small T
    _, r = route(1, 64, 256, 1, 1, 2)
    assert r.partials >= 1
    assert lib.rmsnorm_bwd_workspace_bytes(64, 256, 1, 1) >= r.partials * 256 * 4
    assert route(1, 100, 256, 0, 1, 3)[0] == -3  # no such form


def test_route_recompute_form_has_its_own_launch_shapes():
    """The recompute backward's table: (NV, U, lanes per row, rows per
    block, grid) per width class, as timed in step graphs."""
    want = {(131072, 2048): (2, 2, 128, 2, 512), (4096, 4096): (2, 2, 256, 1, 512),
            (65536, 5120): (4, 1, 192, 2, 256), (1048576, 512): (4, 1, 16, 4, 1024),
            (262144, 1536): (2, 2, 128, 1, 1024), (16384, 6144): (4, 1, 192, 1, 512),
            (8192, 8192): (4, 1, 256, 1, 512), (8192, 16384): (4, 1, 512, 1, 256),
            (786432, 256): (2, 1, 16, 16, 512)}
    for (rows, H), shape in want.items():
        st, r = route(1, rows, H, 0, 1, 2)
        assert st == 0
        assert (r.vec_per_lane, r.unroll, r.lanes_per_row, r.rows_per_block, r.grid) == shape, (rows, H)
        assert r.vec_per_lane * r.lanes_per_row * 8 >= H
        # the workspace query covers the recompute form's partials
        need = lib.rmsnorm_bwd_workspace_bytes(rows, H, 0, 1)
        assert need >= r.partials * H * (8 if r.partial_f64 else 4)


def test_route_plain_backward_launch_shapes():
    """The tuned backward table at each workload: (NV, U, lanes per row,
    row groups per block, grid, FP64 partials, load policy), as timed in
    step graphs on MI355X."""
    want = {
        (4096, 4096, 0, 0): (1, 1, 512, 2, 256, 0, 1),
        (131072, 2048, 1, 0): (1, 1, 256, 4, 256, 1, 2),
        (16384, 6144, 0, 1): (1, 1, 768, 1, 256, 1, 2),
        (786432, 256, 1, 0): (2, 1, 16, 16, 512, 1, 2),
        (131072, 256, 1, 0): (2, 1, 16, 16, 512, 1, 1),
        (1048576, 512, 0, 0): (2, 2, 32, 8, 256, 1, 2),
        (262144, 1536, 1, 0): (1, 1, 192, 4, 256, 1, 2),
        (65536, 5120, 0, 0): (4, 1, 192, 2, 256, 1, 2),
        (8192, 16384, 0, 0): (4, 1, 512, 1, 256, 0, 2),
        (8192, 8192, 0, 0): (1, 1, 1024, 1, 256, 0, 2),
    }
    for (rows, H, wdt, res), shape in want.items():
        st, r = route(1, rows, H, wdt, 1, res)
        assert st == 0
        got = (r.vec_per_lane, r.unroll, r.lanes_per_row, r.rows_per_block, r.grid, r.partial_f64,
               r.stream_loads)
        assert got == shape, (rows, H, got)
        assert r.partials == r.grid and r.block_threads == r.lanes_per_row * r.rows_per_block


def test_route_deterministic_partition_is_a_function_of_shape():
    # same answer for both weight dtypes and for the residual form
    for rows, H in [(4096, 4096), (131072, 2048), (16384, 6144), (786432, 256), (131072, 256)]:
        _, a = route(1, rows, H, 0, 1, 0)
        _, b = route(1, rows, H, 1, 1, 1)
        assert a.grid == b.grid and a.partials == a.grid and a.kind == _lib.RMSN_KIND_BWD_ROW_DET
        # every block owns at least one full iteration of rows
        assert 1 <= a.grid and a.grid * a.rows_per_block * a.unroll <= rows
        ws = lib.rmsnorm_bwd_workspace_bytes(rows, H, 0, 1)
        assert ws >= a.partials * H * (8 if a.partial_f64 else 4)
        assert a.reduce_grid * 16 * (2 if a.partial_f64 else 4) >= H


def test_route_lane_layout_covers_the_row():
    for H in list(range(8, 520, 8)) + [1024, 1032, 1536, 2048, 4096, 5120, 6144, 8192, 12288, 16384]:
        for op in (0, 1):
            for rows in (1, 100, 5000):
                st, r = route(op, rows, H)
                assert st == 0
                nvec = H // 8
                assert r.vec_per_lane * r.lanes_per_row >= nvec
                assert r.block_threads <= 1024 and r.block_threads % 64 == 0 or r.block_threads == 256
                lpr = r.lanes_per_row
                assert (lpr <= 64 and (lpr & (lpr - 1)) == 0) or lpr % 64 == 0
                assert r.rows_per_block * lpr <= r.block_threads
                assert r.grid >= 1


def test_route_rejects_bad_shapes():
    assert route(0, 10, 7)[0] == -3
    assert route(0, 10, 16392)[0] == -3
    assert route(1, -1, 64)[0] == -3
    assert route(1, 10, 64, 3)[0] == -2
    assert route(4, 10, 64)[0] == -3


def test_layernorm_routes():
    # the backward runs the row kernel and the [P, 2H] partial reduce at every T
    for rows in (1, 64, 65, 8192, 8193, 262144):
        for H in (256, 512, 2048, 3584, 4096, 8192, 16384):
            st, r = route(3, rows, H, 0, 1)
            assert st == 0 and r.kind == _lib.RMSN_KIND_BWD_ROW_DET
            assert r.partials == r.grid >= 1
            assert r.partial_f64 == (1 if rows > 8192 else 0)
            need = lib.layernorm_bwd_workspace_bytes(rows, H, 0, 1)
            assert need >= r.partials * 2 * H * (8 if r.partial_f64 else 4)
            assert r.reduce_grid * 16 * (2 if r.partial_f64 else 4) >= 2 * H
            assert r.vec_per_lane * r.lanes_per_row >= H // 8
            st, f = route(2, rows, H, 0, 1)
            assert st == 0 and f.kind == _lib.RMSN_KIND_FWD_ROW
            assert f.vec_per_lane * f.lanes_per_row >= H // 8


def test_route_override_selects_atomic_and_rejects_bad_knobs():
    K = _lib.RouteKnobs
    _, before = route(0, 4096, 256)
    try:
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(0, 0, 0, 0, 0, _lib.RMSN_KIND_BWD_ROW_ATOMIC))) == 0
        st, r = route(1, 131072, 2048, 1, 0)
        assert st == 0 and r.kind == _lib.RMSN_KIND_BWD_ROW_ATOMIC and r.partials == 0
        st, r = route(1, 131072, 2048, 1, 1)  # deterministic calls ignore the kind knob
        assert st == 0 and r.kind == _lib.RMSN_KIND_BWD_ROW_DET
        assert lib.rmsnorm_bwd_workspace_bytes(131072, 2048, 1, 0) >= 2048 * 8 + 4
        # knobs the kernels cannot honour make the route fail (no launch)
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(3, 0, 0, 0, 0, 0))) == 0
        assert route(1, 131072, 2048, 1, 1)[0] == -3
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(4, 2, 0, 0, 0, 0))) == 0
        assert route(1, 4096, 16384, 1, 1)[0] == -3    # backward NV 4 is compiled for U = 1
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(4, 1, 0, 0, 0, 0))) == 0
        st, r = route(1, 4096, 16384, 1, 1)
        assert st == 0 and r.vec_per_lane == 4 and r.lanes_per_row == 512
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(2, 8, 0, 0, 0, 0))) == 0
        assert route(1, 4096, 4096, 0, 1)[0] == -3     # NV * U > 8 is not compiled
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(1, 8, 1, 0, 0, 0))) == 0
        assert route(1, 4096, 4096, 0, 1)[0] == -3     # backward NV * U > 4 is not compiled
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(1, 2, 2, 0, 0, 0))) == 0
        assert route(1, 4096, 4096, 0, 1)[0] == -3     # wide rows, NV * U >= 2: <= 512 threads
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(1, 2, 1, 0, 0, 0))) == 0
        st, r = route(1, 4096, 4096, 0, 1)
        assert st == 0 and r.block_threads == 512
        assert lib.rmsnorm_route_override(3, ctypes.byref(K(2, 1, 8, 0, 0, 0))) == 0
        assert route(3, 4096, 2048, 0, 1)[0] == -3     # LayerNorm backward: the same bound
        assert lib.rmsnorm_route_override(3, ctypes.byref(K(2, 1, 4, 0, 0, 0))) == 0
        st, r = route(3, 4096, 2048, 0, 1)
        assert st == 0 and r.block_threads == 512
        assert lib.rmsnorm_route_override(0, ctypes.byref(K(1, 8, 1, 0, 0, 0))) == 0
        assert route(0, 4096, 4096)[0] == 0             # the forward keeps NV * U = 8
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(2, 4, 0, 0, 0, 3))) == 0
        assert route(1, 4096, 4096, 0, 0)[0] == -3     # atomic variant compiled for NV 1, U <= 2
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(1, 0, 64, 0, 0, 0))) == 0
        assert route(1, 4096, 256, 0, 1)[0] == -3      # 64 x 32 lanes > 256 threads
        assert lib.rmsnorm_route_override(1, ctypes.byref(K(0, 0, 0, 99, 0, 0))) == -3
        assert lib.rmsnorm_route_override(0, ctypes.byref(K(4, 4, 0, 0, 0, 0))) == 0
        assert route(0, 4096, 4096)[0] == -3
        assert lib.rmsnorm_route_override(0, ctypes.byref(K(1, 4, 0, 0, 0, 0))) == 0
        st, r = route(0, 4096, 256)
        assert st == 0 and r.unroll == 4 and r.vec_per_lane == 1
    finally:
        lib.rmsnorm_route_override(0, None)
        lib.rmsnorm_route_override(1, None)
        lib.rmsnorm_route_override(3, None)
    st, r = route(0, 4096, 256)
    assert st == 0 and (r.unroll, r.vec_per_lane, r.grid) == (before.unroll, before.vec_per_lane, before.grid)


def test_route_stream_loads_policy_follows_shape():
    """Non-temporal loads in the RMSNorm backward: 1 (dy/dres streamed)
    below a forward footprint of 256 MiB (the Infinity Cache), 2 (every
    input) from there on; the residual form counts four tensors in the
    forward, the plain form two. LayerNorm's backward streams nothing below
    32M elements. The forward streams only the residual form's x and r, at
    level 2; LayerNorm's forward never (its backward reads x again)."""
    MiE = 1024 * 1024
    b = lambda *a: route(1, *a)[1].stream_loads
    f = lambda *a: route(0, *a)[1].stream_loads
    assert b(4096, 4096) == 1                       # 16M elements
    assert b(65, 256) == 1
    assert b(32768 * 4, 256, 1) == 1                # 32M, 128 MiB forward
    assert b(32768 * 4, 256, 1, 1, 1) == 2          # residual: 256 MiB
    assert b(32768 * 4 - 1, 256, 1, 1, 1) == 1      # just under
    assert b(131072, 2048, 1) == 2
    assert b(32768 * 24, 256, 1) == 2
    assert b(16384, 6144, 0, 1, 1) == 2
    assert b(32 * MiE // 4096 - 1, 4096) == 1
    assert route(1, 4096, 4096, 0, 1, 2)[1].stream_loads == 1   # recompute form
    for shape in [(4096, 4096), (32768 * 4, 256, 1), (131072, 2048, 1), (32768 * 24, 256, 1)]:
        assert f(*shape) == 0                       # plain forward: x is read again
    assert f(16384, 6144, 0, 1, 1) == 2             # residual forward, 768 MiB
    assert f(32768 * 4, 256, 1, 1, 1) == 2
    assert f(32768 * 2, 256, 1, 1, 1) == 0          # residual, 128 MiB
    # the column-task path does not use it; LayerNorm: backward as RMSNorm's
    assert route(1, 64, 256, 1)[1].stream_loads == 0
    assert route(2, 8192, 8192)[1].stream_loads == 0
    assert route(3, 8192, 3584)[1].stream_loads == 0
    assert route(3, 8192, 4096)[1].stream_loads == 1
    assert route(3, 8192, 8192)[1].stream_loads == 2
    K = _lib.RouteKnobs
    try:
        k = K(); k.stream_loads = 3
        assert lib.rmsnorm_route_override(1, ctypes.byref(k)) == 0
        assert route(1, 4096, 4096)[1].stream_loads == 2
        assert lib.rmsnorm_route_override(0, ctypes.byref(k)) == 0
        assert route(0, 131072, 2048)[1].stream_loads == 2
        k.stream_loads = 1
        assert lib.rmsnorm_route_override(1, ctypes.byref(k)) == 0
        assert route(1, 131072, 2048, 1)[1].stream_loads == 0
        k.stream_loads = 4
        assert lib.rmsnorm_route_override(1, ctypes.byref(k)) == -3
    finally:
        lib.rmsnorm_route_override(0, None)
        lib.rmsnorm_route_override(1, None)


def test_loader_refuses_a_library_built_from_other_sources(tmp_path, monkeypatch):
    """The binding's structs must match the library's: a build whose recorded
    code hash differs from the sources is refused before it is loaded."""
    stale = tmp_path / "libbwd_rmsnorm.hash"
    stale.write_text("0000000000000000\n")
    monkeypatch.setattr(_lib, "HASH_PATH", str(stale))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="built from other sources"):
        _lib.load()


def test_code_hash_ignores_comments_and_layout():
    from bwd_rmsnorm_fwd_02_amd import build
    a = "int f(int x) { // note\n  return x + 1; /* more */ }\n"
    b = "int f(int x) {\n\n    return x + 1;   }"
    c = "int f(int x) { return x + 2; }"
    s = 'const char* s = "// kept";'
    assert build._code_only(a) == build._code_only(b)
    assert build._code_only(a) != build._code_only(c)
    assert "// kept" in build._code_only(s)
