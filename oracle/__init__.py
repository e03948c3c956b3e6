"""FP64 CPU oracle for RMSNorm training (ctypes wrapper over rmsnorm_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module. The HIP
library never loads it, and it shares no source with the HIP library.

It computes the plain definition of RMSNorm forward and backward in double
precision (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
backward routes", opening description and "Key"/"Workload" paragraphs):

* ``fwd``: rstd = 1/sqrt(mean(x^2) + eps), y = x*rstd*w
* ``bwd``: dx = rstd*(dy*w - xhat*c), c = mean(dy*w*xhat), dw = sum_t dy*xhat
* ``residual_add``: h = BF16(x + r)
* ``ln_fwd`` / ``ln_bwd``: LayerNorm, the adjacent normalisation of the same
  benchmark suite (ROCm TransformerEngine PR "Microbenchmarking and CI
  performance regression test", benchmark_normalization): mu = mean(x),
  var = mean((x - mu)^2), rstd = 1/sqrt(var + eps),
  y = (x - mu)*rstd*gamma + beta; dx = rstd*(g - mean(g) - xhat*mean(g*xhat))
  with g = dy*gamma, dgamma = sum_t dy*xhat, dbeta = sum_t dy

Inputs are BF16 bit patterns (numpy ``uint16``) for x, dy, r, and float64 for
w and rstd. All arrays are contiguous ``[rows, H]``; per-head views are
flattened by the caller (row = t * heads + head).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmsnorm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.orc_bf16_to_double.argtypes = [i64, p, p]
    lib.orc_round_bf16.argtypes = [i64, p, p]
    lib.orc_round_f32.argtypes = [i64, p, p]
    lib.orc_fwd.argtypes = [i64, i64, p, p, ctypes.c_double, p, p]
    lib.orc_bwd.argtypes = [i64, i64, p, p, p, p, p, p, p]
    lib.orc_residual_add.argtypes = [i64, p, p, p]
    lib.orc_fwd_f64.argtypes = [i64, i64, p, p, ctypes.c_double, p, p]
    lib.orc_bwd_f64.argtypes = [i64, i64, p, p, p, p, p, p, p]
    lib.orc_ln_fwd.argtypes = [i64, i64, p, p, p, ctypes.c_double, p, p, p]
    lib.orc_ln_bwd.argtypes = [i64, i64, p, p, p, p, p, p, p, p, p]
    lib.orc_ln_fwd_f64.argtypes = [i64, i64, p, p, p, ctypes.c_double, p, p, p]
    lib.orc_ln_bwd_f64.argtypes = [i64, i64, p, p, p, p, p, p, p, p, p]
    for f in (lib.orc_bf16_to_double, lib.orc_round_bf16, lib.orc_round_f32,
              lib.orc_fwd, lib.orc_bwd, lib.orc_residual_add,
              lib.orc_fwd_f64, lib.orc_bwd_f64, lib.orc_ln_fwd, lib.orc_ln_bwd,
              lib.orc_ln_fwd_f64, lib.orc_ln_bwd_f64):
        f.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def bf16_to_double(bits: np.ndarray) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().orc_bf16_to_double(bits.size, _ptr(bits), _ptr(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (nearest-even, one rounding); bit patterns."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_round_bf16(v.size, _ptr(v), _ptr(out))
    return out


def round_f32(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.float32)
    _load().orc_round_f32(v.size, _ptr(v), _ptr(out))
    return out


def fwd(x_bits: np.ndarray, w: np.ndarray, eps: float, want_y: bool = True):
    """Forward over rows of x. Returns (rstd[rows], y[rows, H] or None) in float64."""
    x_bits = _c(x_bits, np.uint16)
    rows, H = x_bits.shape
    w = _c(w, np.float64)
    assert w.shape == (H,)
    rstd = np.empty(rows, np.float64)
    y = np.empty((rows, H), np.float64) if want_y else None
    _load().orc_fwd(rows, H, _ptr(x_bits), _ptr(w), float(eps), _ptr(rstd), _ptr(y))
    return rstd, y


def bwd(dy_bits: np.ndarray, x_bits: np.ndarray, rstd: np.ndarray, w: np.ndarray,
        want_dx: bool = True):
    """Backward at the given rstd. Returns (dx or None, c or None, dw), float64."""
    dy_bits = _c(dy_bits, np.uint16)
    x_bits = _c(x_bits, np.uint16)
    rows, H = x_bits.shape
    assert dy_bits.shape == (rows, H)
    rstd = _c(rstd, np.float64)
    assert rstd.shape == (rows,)
    w = _c(w, np.float64)
    assert w.shape == (H,)
    dx = np.empty((rows, H), np.float64) if want_dx else None
    c = np.empty(rows, np.float64) if want_dx else None
    dw = np.empty(H, np.float64)
    _load().orc_bwd(rows, H, _ptr(dy_bits), _ptr(x_bits), _ptr(rstd), _ptr(w),
                    _ptr(dx), _ptr(c), _ptr(dw))
    return dx, c, dw


def fwd_f64(x: np.ndarray, w: np.ndarray, eps: float):
    """Forward on unrounded float64 rows (same per-row code as ``fwd``)."""
    x = _c(x, np.float64)
    rows, H = x.shape
    w = _c(w, np.float64)
    rstd = np.empty(rows, np.float64)
    y = np.empty((rows, H), np.float64)
    _load().orc_fwd_f64(rows, H, _ptr(x), _ptr(w), float(eps), _ptr(rstd), _ptr(y))
    return rstd, y


def bwd_f64(dy: np.ndarray, x: np.ndarray, rstd: np.ndarray, w: np.ndarray):
    """Backward on unrounded float64 rows (same per-row code as ``bwd``)."""
    dy = _c(dy, np.float64)
    x = _c(x, np.float64)
    rows, H = x.shape
    rstd = _c(rstd, np.float64)
    w = _c(w, np.float64)
    dx = np.empty((rows, H), np.float64)
    c = np.empty(rows, np.float64)
    dw = np.empty(H, np.float64)
    _load().orc_bwd_f64(rows, H, _ptr(dy), _ptr(x), _ptr(rstd), _ptr(w),
                        _ptr(dx), _ptr(c), _ptr(dw))
    return dx, c, dw


def residual_add(x_bits: np.ndarray, r_bits: np.ndarray) -> np.ndarray:
    x_bits = _c(x_bits, np.uint16)
    r_bits = _c(r_bits, np.uint16)
    assert x_bits.shape == r_bits.shape
    h = np.empty(x_bits.shape, np.uint16)
    _load().orc_residual_add(x_bits.size, _ptr(x_bits), _ptr(r_bits), _ptr(h))
    return h


# ------------------------------------------------------------------ LayerNorm

def _ln_params(H, gamma, beta):
    gamma = _c(gamma, np.float64)
    assert gamma.shape == (H,)
    if beta is not None:
        beta = _c(beta, np.float64)
        assert beta.shape == (H,)
    return gamma, beta


def ln_fwd(x_bits: np.ndarray, gamma: np.ndarray, beta, eps: float, want_y: bool = True):
    """LayerNorm forward over rows of x (BF16 bits). beta may be None (zero).
    Returns (mu[rows], rstd[rows], y[rows, H] or None), float64."""
    x_bits = _c(x_bits, np.uint16)
    rows, H = x_bits.shape
    gamma, beta = _ln_params(H, gamma, beta)
    mu = np.empty(rows, np.float64)
    rstd = np.empty(rows, np.float64)
    y = np.empty((rows, H), np.float64) if want_y else None
    _load().orc_ln_fwd(rows, H, _ptr(x_bits), _ptr(gamma), _ptr(beta), float(eps),
                       _ptr(mu), _ptr(rstd), _ptr(y))
    return mu, rstd, y


def ln_bwd(dy_bits: np.ndarray, x_bits: np.ndarray, mu: np.ndarray, rstd: np.ndarray,
           gamma: np.ndarray, want_dx: bool = True):
    """LayerNorm backward at the given mu and rstd. Returns
    (dx or None, c[rows, 2] = (c1, c2) or None, dgamma, dbeta), float64."""
    dy_bits = _c(dy_bits, np.uint16)
    x_bits = _c(x_bits, np.uint16)
    rows, H = x_bits.shape
    assert dy_bits.shape == (rows, H)
    mu = _c(mu, np.float64)
    rstd = _c(rstd, np.float64)
    assert mu.shape == (rows,) and rstd.shape == (rows,)
    gamma, _ = _ln_params(H, gamma, None)
    dx = np.empty((rows, H), np.float64) if want_dx else None
    c = np.empty((rows, 2), np.float64) if want_dx else None
    dg = np.empty(H, np.float64)
    db = np.empty(H, np.float64)
    _load().orc_ln_bwd(rows, H, _ptr(dy_bits), _ptr(x_bits), _ptr(mu), _ptr(rstd), _ptr(gamma),
                       _ptr(dx), _ptr(c), _ptr(dg), _ptr(db))
    return dx, c, dg, db


def ln_fwd_f64(x: np.ndarray, gamma: np.ndarray, beta, eps: float):
    """LayerNorm forward on unrounded float64 rows (same per-row code)."""
    x = _c(x, np.float64)
    rows, H = x.shape
    gamma, beta = _ln_params(H, gamma, beta)
    mu = np.empty(rows, np.float64)
    rstd = np.empty(rows, np.float64)
    y = np.empty((rows, H), np.float64)
    _load().orc_ln_fwd_f64(rows, H, _ptr(x), _ptr(gamma), _ptr(beta), float(eps),
                           _ptr(mu), _ptr(rstd), _ptr(y))
    return mu, rstd, y


def ln_bwd_f64(dy: np.ndarray, x: np.ndarray, mu: np.ndarray, rstd: np.ndarray,
               gamma: np.ndarray):
    """LayerNorm backward on unrounded float64 rows (same per-row code)."""
    dy = _c(dy, np.float64)
    x = _c(x, np.float64)
    rows, H = x.shape
    mu = _c(mu, np.float64)
    rstd = _c(rstd, np.float64)
    gamma, _ = _ln_params(H, gamma, None)
    dx = np.empty((rows, H), np.float64)
    c = np.empty((rows, 2), np.float64)
    dg = np.empty(H, np.float64)
    db = np.empty(H, np.float64)
    _load().orc_ln_bwd_f64(rows, H, _ptr(dy), _ptr(x), _ptr(mu), _ptr(rstd), _ptr(gamma),
                           _ptr(dx), _ptr(c), _ptr(dg), _ptr(db))
    return dx, c, dg, db
