"""Element-by-element comparison of whole full-size outputs with the oracle.

The full-size parity tests compare every row of y, dx (dh) and, for
LayerNorm, of both outputs, not a sample: the rows are cut into chunks of
about 256K elements (small enough that each chunk's temporaries stay in the
allocator's reuse range, measured fastest), and each chunk is recomputed by the oracle and
checked against the GPU result on a pool of host threads (the oracle's C
code and numpy's array operations run outside the interpreter lock). Output
buffers are filled with a NaN pattern before the GPU call, so an element the
kernel never writes fails the comparison.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle
from tests.parity import (check_bf16_strict, check_dx, dx_bound, ln_dx_bound, ln_y_bound,
                          to_f64)

# BF16 quiet NaN: the fill of every output before a GPU call
SENTINEL = 0x7FC0
THREADS = min(16, os.cpu_count() or 1)


def row_chunks(rows: int, H: int, target: int = 1 << 18):
    step = max(1, target // max(H, 1))
    return [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]


def map_rows(fn, rows: int, H: int):
    """fn(lo, hi) over row chunks on the thread pool; results in chunk order.
    An assertion raised in any chunk propagates."""
    chunks = row_chunks(rows, H)
    if len(chunks) == 1:
        return [fn(*chunks[0])]
    with cf.ThreadPoolExecutor(max_workers=THREADS) as ex:
        return list(ex.map(lambda b: fn(*b), chunks))


def check_y_rows(name, y_bits, x_bits, w64, eps):
    """y within one BF16 ulp of RNE(y64) on every element of every row."""
    rows, H = x_bits.shape

    def one(lo, hi):
        _, y64 = oracle.fwd(x_bits[lo:hi], w64, eps)
        check_bf16_strict(f"{name} rows [{lo}, {hi})", y_bits[lo:hi], y64)

    map_rows(one, rows, H)


def check_dx_rows(name, dx_bits, dy_bits, x_bits, rstd64, w64, dres_bits=None) -> int:
    """dx (dh = dx + dres in the residual form) on every row against the
    oracle at the given rstd, with the cancellation exemption. Returns the
    number of exempted elements."""
    rows, H = x_bits.shape

    def one(lo, hi):
        dx64, c64, _ = oracle.bwd(dy_bits[lo:hi], x_bits[lo:hi], rstd64[lo:hi], w64)
        dres64 = to_f64(dres_bits[lo:hi]) if dres_bits is not None else None
        E = dx_bound(to_f64(x_bits[lo:hi]), to_f64(dy_bits[lo:hi]), w64, rstd64[lo:hi], c64, H,
                     dres64)
        ref = dx64 + dres64 if dres64 is not None else dx64
        return check_dx(f"{name} rows [{lo}, {hi})", dx_bits[lo:hi], ref, E)

    return int(sum(map_rows(one, rows, H)))


def check_ln_y_rows(name, y_bits, x_bits, mu64, rs64, g64, b64, eps) -> int:
    rows, H = x_bits.shape

    def one(lo, hi):
        _, _, y64 = oracle.ln_fwd(x_bits[lo:hi], g64, b64, eps)
        E = ln_y_bound(to_f64(x_bits[lo:hi]), mu64[lo:hi], rs64[lo:hi], g64, b64)
        return check_dx(f"{name} rows [{lo}, {hi})", y_bits[lo:hi], y64, E)

    return int(sum(map_rows(one, rows, H)))


def check_ln_dx_rows(name, dx_bits, dy_bits, x_bits, mu32, rs32, g64) -> int:
    rows, H = x_bits.shape

    def one(lo, hi):
        dx64, c64, _, _ = oracle.ln_bwd(dy_bits[lo:hi], x_bits[lo:hi], mu32[lo:hi], rs32[lo:hi], g64)
        E = ln_dx_bound(to_f64(x_bits[lo:hi]), to_f64(dy_bits[lo:hi]), g64, mu32[lo:hi],
                        rs32[lo:hi], c64, H)
        return check_dx(f"{name} rows [{lo}, {hi})", dx_bits[lo:hi], dx64, E)

    return int(sum(map_rows(one, rows, H)))


def unwritten(bits: np.ndarray) -> int:
    """Elements still holding the fill pattern."""
    return int(np.count_nonzero(bits == SENTINEL))
