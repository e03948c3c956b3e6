"""Pins for the FP64 oracle: it is checked against things other than itself.

Each test checks the oracle against a fact the pages or the mathematics fix,
so that a plausible mistake in it (a dropped term, a wrong sign or index, a
transposed operand, a double rounding) fails at least one of them:

* BF16 rounding: against torch's float32->bfloat16 conversion, against exact
  rational rounding over the full BF16 grid, and against hand-derived ties,
  overflow and subnormal cases;
* forward and backward: central finite differences of L = sum(y * dy) with
  respect to x and w, and torch autograd through ``torch.nn.functional.rms_norm``
  in float64 on the CPU (a library routine);
* closed forms (constant, zero and single-element rows, T = 1, dy = 1),
  power-of-two scale invariance, the orthogonality of dx to x, linearity in
  dy, dy = 0;
* dw against an exact rational sum on small T, and row-permutation invariance;
* the residual pre-add against float32 addition plus torch's rounding.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import synth

EPS = 1e-6


# ---------------------------------------------------------------- BF16 rounding

def _all_finite_bf16():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    vals = synth.bits_to_f32(bits).astype(np.float64)
    return bits, vals


_POS_BITS, _POS_VALS = _all_finite_bf16()
_POS_FRAC = [Fraction(float(v)) for v in _POS_VALS]


def _exact_round_bf16(v: float) -> int:
    """Nearest BF16 to v (ties to even mantissa) by search over the full grid."""
    if v != v:
        raise ValueError
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = Fraction(abs(v))
    maxv = _POS_FRAC[-1]
    # next grid point after the largest finite value would be 2^128
    if a >= (maxv + Fraction(2) ** 128) / 2:
        return sign | 0x7F80
    i = bisect.bisect_left(_POS_FRAC, a)
    if i < len(_POS_FRAC) and _POS_FRAC[i] == a:
        return sign | int(_POS_BITS[i])
    lo, hi = i - 1, i
    if hi >= len(_POS_FRAC):
        return sign | int(_POS_BITS[lo])
    dlo, dhi = a - _POS_FRAC[lo], _POS_FRAC[hi] - a
    if dlo < dhi:
        k = lo
    elif dhi < dlo:
        k = hi
    else:
        k = lo if (int(_POS_BITS[lo]) & 1) == 0 else hi
    return sign | int(_POS_BITS[k])


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
        (rng.standard_normal(50000) * 1e-38).astype(np.float32),  # subnormal range
        # exact ties: BF16 value plus half its ulp
        (synth.bits_to_f32(np.arange(0x3F80, 0x4080, dtype=np.uint16))
         * np.float32(1 + 2 ** -8)).astype(np.float32),
    ])
    ours = oracle.round_bf16(a.astype(np.float64))
    ref = synth.bf16_bits(a)
    assert np.array_equal(ours, ref)


def test_round_bf16_single_rounding_from_double():
    rng = np.random.default_rng(2)
    # doubles with more than 24 significant bits, so a route through float32
    # would round twice
    base = synth.bits_to_f32(rng.integers(0x0001, 0x7F7F, 3000).astype(np.uint16)).astype(np.float64)
    frac = rng.integers(1, 2 ** 20, 3000) * 2.0 ** -28
    vals = base * (1.0 + 2.0 ** -8 + frac * 2.0 ** -8 * (rng.integers(0, 2, 3000) * 2 - 1))
    vals = np.concatenate([vals, -vals[:500]])
    ours = oracle.round_bf16(vals)
    for v, o in zip(vals, ours):
        assert int(o) == _exact_round_bf16(float(v)), v


@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),            # tie -> even (1.0)
    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie -> even (1 + 2^-6)
    (1.0 + 2 ** -8 + 2 ** -40, 0x3F81),  # just above the tie
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),          # largest finite
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),          # tie at the top -> inf
    ((2 - 2 ** -8 - 2 ** -20) * 2.0 ** 127, 0x7F7F),
    (2.0 ** -133, 0x0001),              # smallest subnormal
    (2.0 ** -134, 0x0000),              # tie -> even (0)
    (3 * 2.0 ** -134, 0x0002),          # tie -> even (2 quanta)
    (2.0 ** -126, 0x0080),              # smallest normal
    (math.inf, 0x7F80),
    (-math.inf, 0xFF80),
])
def test_round_bf16_hand_cases(v, bits):
    assert int(oracle.round_bf16(np.array([v]))[0]) == bits


def test_round_bf16_nan():
    out = int(oracle.round_bf16(np.array([math.nan]))[0])
    assert (out & 0x7F80) == 0x7F80 and (out & 0x007F) != 0


def test_widening_is_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_double(bits)
    ref = synth.bits_to_f32(bits).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


# --------------------------------------------------- forward / backward formulas

def _loss(x, w, dy, eps):
    _, y = oracle.fwd_f64(x, w, eps)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("T,H,eps", [(1, 1, 0.3), (2, 5, EPS), (3, 8, 0.05), (3, 7, 1e-3)])
def test_backward_matches_finite_differences(T, H, eps):
    rng = np.random.default_rng(10 + H)
    x = rng.standard_normal((T, H))
    w = 1 + 0.3 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    rstd, _ = oracle.fwd_f64(x, w, eps)
    dx, _, dw = oracle.bwd_f64(dy, x, rstd, w)
    h = 1e-5
    fd_x = np.empty_like(x)
    for t in range(T):
        for j in range(H):
            xp, xm = x.copy(), x.copy()
            xp[t, j] += h
            xm[t, j] -= h
            fd_x[t, j] = (_loss(xp, w, dy, eps) - _loss(xm, w, dy, eps)) / (2 * h)
    fd_w = np.empty_like(w)
    for j in range(H):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        fd_w[j] = (_loss(x, wp, dy, eps) - _loss(x, wm, dy, eps)) / (2 * h)
    scale_x = np.max(np.abs(fd_x)) + 1e-30
    scale_w = np.max(np.abs(fd_w)) + 1e-30
    assert np.max(np.abs(dx - fd_x)) / scale_x < 1e-7
    assert np.max(np.abs(dw - fd_w)) / scale_w < 1e-7


@pytest.mark.parametrize("T,H,eps", [(4, 16, EPS), (7, 64, 0.01), (3, 256, EPS)])
def test_matches_torch_rms_norm_autograd_float64(T, H, eps):
    rng = np.random.default_rng(20 + H)
    x = rng.standard_normal((T, H))
    w = 1 + 0.1 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    yt = torch.nn.functional.rms_norm(xt, (H,), wt, eps)
    yt.backward(torch.tensor(dy, dtype=torch.float64))
    rstd, y = oracle.fwd_f64(x, w, eps)
    dx, _, dw = oracle.bwd_f64(dy, x, rstd, w)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_closed_form_rows():
    # [3, 4] with eps 0: mean square 12.5
    rstd, y = oracle.fwd_f64(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    assert rstd[0] == 1.0 / math.sqrt(12.5)
    assert y[0, 0] == 3.0 * rstd[0] and y[0, 1] == (4.0 * rstd[0]) * 2.0
    # constant row c = 2 (BF16 bits 0x4000)
    x = np.full((1, 8), 0x4000, np.uint16)
    rstd, _ = oracle.fwd(x, np.ones(8), EPS)
    assert rstd[0] == 1.0 / math.sqrt(4.0 + EPS)
    # zero row: 1/sqrt(eps)
    rstd, y = oracle.fwd(np.zeros((1, 16), np.uint16), np.ones(16), EPS)
    assert rstd[0] == 1.0 / math.sqrt(EPS) and np.all(y == 0)
    # H = 1: xhat = x / sqrt(x^2 + eps)
    rstd, y = oracle.fwd_f64(np.array([[-1.75]]), np.array([1.0]), 0.25)
    assert y[0, 0] == -1.75 * (1.0 / math.sqrt(1.75 ** 2 + 0.25))


def test_power_of_two_scale_invariance_bitwise():
    wl = synth.make(T=32, H=512, w_dtype="f32", seed=3)
    x = oracle.bf16_to_double(wl.x)
    rstd1, y1 = oracle.fwd_f64(x, wl.w.f64, 0.0)
    rstd8, y8 = oracle.fwd_f64(8.0 * x, wl.w.f64, 0.0)
    assert np.array_equal(rstd8 * 8.0, rstd1)
    assert np.array_equal(y8, y1)


@pytest.mark.parametrize("eps", [0.0, 0.5])
def test_dx_orthogonal_to_x(eps):
    rng = np.random.default_rng(4)
    T, H = 16, 96
    x = rng.standard_normal((T, H))
    w = 1 + 0.1 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    rstd, _ = oracle.fwd_f64(x, w, eps)
    dx, _, _ = oracle.bwd_f64(dy, x, rstd, w)
    ms = np.mean(x * x, axis=1)
    gx = np.sum(dy * w * x, axis=1)
    expect = rstd * (eps / (ms + eps)) * gx
    got = np.sum(x * dx, axis=1)
    scale = np.sum(np.abs(x * dx), axis=1)
    assert np.all(np.abs(got - expect) <= 1e-13 * scale)
    if eps > 0:
        assert np.all(np.abs(expect) > 1e-3 * scale)  # the case is not trivial


def test_linear_in_dy_and_zero_dy():
    rng = np.random.default_rng(5)
    T, H = 9, 40
    x = rng.standard_normal((T, H))
    w = 1 + 0.1 * rng.standard_normal(H)
    d1, d2 = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    rstd, _ = oracle.fwd_f64(x, w, EPS)
    a, b = 0.75, -2.5
    dxa, _, dwa = oracle.bwd_f64(a * d1 + b * d2, x, rstd, w)
    dx1, _, dw1 = oracle.bwd_f64(d1, x, rstd, w)
    dx2, _, dw2 = oracle.bwd_f64(d2, x, rstd, w)
    np.testing.assert_allclose(dxa, a * dx1 + b * dx2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dwa, a * dw1 + b * dw2, rtol=1e-12, atol=1e-12)
    dx0, c0, dw0 = oracle.bwd_f64(np.zeros((T, H)), x, rstd, w)
    assert np.all(dx0 == 0) and np.all(dw0 == 0) and np.all(c0 == 0)


def test_dw_single_row_and_unit_dy():
    wl = synth.make(T=1, H=64, w_dtype="bf16", seed=6)
    rstd, _ = oracle.fwd(wl.x, wl.w.f64, EPS, want_y=False)
    _, _, dw = oracle.bwd(wl.dy, wl.x, rstd, wl.w.f64)
    x = oracle.bf16_to_double(wl.x)
    dy = oracle.bf16_to_double(wl.dy)
    assert np.array_equal(dw, dy[0] * (x[0] * rstd[0]))
    # dy = 1 everywhere: dw_j = sum_t xhat_tj
    wl = synth.make(T=50, H=32, w_dtype="f32", seed=7)
    ones = np.full(wl.x.shape, 0x3F80, np.uint16)
    rstd, _ = oracle.fwd(wl.x, wl.w.f64, EPS, want_y=False)
    _, _, dw = oracle.bwd(ones, wl.x, rstd, wl.w.f64)
    xhat = oracle.bf16_to_double(wl.x) * rstd[:, None]
    assert np.allclose(dw, [math.fsum(xhat[:, j]) for j in range(32)], rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("T,H,wdt", [(512, 8, "bf16"), (2048, 4, "f32")])
def test_dw_against_exact_rational_sum(T, H, wdt):
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=8, heavy_frac=0.02)
    rstd, _ = oracle.fwd(wl.x, wl.w.f64, EPS, want_y=False)
    _, _, dw = oracle.bwd(wl.dy, wl.x, rstd, wl.w.f64)
    x = oracle.bf16_to_double(wl.x)
    dy = oracle.bf16_to_double(wl.dy)
    u = 2.0 ** -53
    for j in range(H):
        terms = [Fraction(float(dy[t, j])) * Fraction(float(x[t, j])) * Fraction(float(rstd[t]))
                 for t in range(T)]
        exact = sum(terms, Fraction(0))
        mag = float(sum(abs(q) for q in terms))
        err = abs(Fraction(float(dw[j])) - exact)
        # two product roundings per term plus the final rounding of the sum
        assert float(err) <= 2.5 * u * mag + u * abs(float(exact)), (j, float(err))


def test_dw_row_permutation_invariance():
    wl = synth.make(T=3000, H=24, w_dtype="f32", seed=9)
    rstd, _ = oracle.fwd(wl.x, wl.w.f64, EPS, want_y=False)
    _, _, dw = oracle.bwd(wl.dy, wl.x, rstd, wl.w.f64)
    p = np.random.default_rng(0).permutation(3000)
    _, _, dwp = oracle.bwd(wl.dy[p], wl.x[p], rstd[p], wl.w.f64)
    np.testing.assert_allclose(dw, dwp, rtol=1e-14, atol=1e-13)


def test_bf16_and_f64_entry_points_agree():
    wl = synth.make(T=20, H=48, w_dtype="bf16", seed=11)
    r1, y1 = oracle.fwd(wl.x, wl.w.f64, EPS)
    x = oracle.bf16_to_double(wl.x)
    r2, y2 = oracle.fwd_f64(x, wl.w.f64, EPS)
    assert np.array_equal(r1, r2) and np.array_equal(y1, y2)
    dx1, c1, dw1 = oracle.bwd(wl.dy, wl.x, r1, wl.w.f64)
    dx2, c2, dw2 = oracle.bwd_f64(oracle.bf16_to_double(wl.dy), x, r1, wl.w.f64)
    assert np.array_equal(dx1, dx2) and np.array_equal(c1, c2) and np.array_equal(dw1, dw2)
    _, _, dw3 = oracle.bwd(wl.dy, wl.x, r1, wl.w.f64, want_dx=False)
    assert np.array_equal(dw1, dw3)


def test_residual_add_matches_float32_sum_and_torch_rounding():
    rng = np.random.default_rng(12)
    x = synth.normal_bf16(rng, 100000)
    r = synth.normal_bf16(rng, 100000)
    # include wide exponent gaps and exact cancellations
    r[:1000] = synth.bf16_bits(synth.bits_to_f32(x[:1000]) * np.float32(-1.0))
    r[1000:2000] = synth.bf16_bits(synth.bits_to_f32(r[1000:2000]) * np.float32(2.0 ** -30))
    h = oracle.residual_add(x, r)
    ref = synth.bf16_bits(synth.bits_to_f32(x) + synth.bits_to_f32(r))
    assert np.array_equal(h, ref)
    for i in range(2000, 2200):
        exact = float(synth.bits_to_f32(x[i:i + 1])[0]) + float(synth.bits_to_f32(r[i:i + 1])[0])
        assert int(h[i]) == _exact_round_bf16(exact)


def test_non_finite_inputs_propagate_as_ieee_arithmetic_fixes():
    """Non-finite inputs are not special-cased: a row holding +inf has an
    infinite sum of squares, so rstd = 1/sqrt(inf) = 0 exactly, xhat = inf * 0
    is NaN at that element and 0 elsewhere; its c is NaN, so its dx is NaN
    throughout, and dw is NaN only in that column. A NaN in dy spoils its
    row's dx and its own column of dw; a NaN in x spoils its row (rstd, y,
    dx) and every column of dw."""
    H, T = 16, 4
    w = 1.0 + 0.1 * np.arange(H)
    x = synth.bf16_bits(np.linspace(-2, 2, T * H, dtype=np.float32).reshape(T, H))
    dy = synth.bf16_bits(np.linspace(1, -1, T * H, dtype=np.float32).reshape(T, H))
    x[1, 3] = 0x7F80   # +inf
    dy[2, 7] = 0x7FC0  # NaN
    rstd, y = oracle.fwd(x, w, EPS)
    assert rstd[1] == 0.0 and np.isfinite(rstd[[0, 2, 3]]).all()
    assert np.isnan(y[1, 3]) and np.all(y[1, np.arange(H) != 3] == 0.0)
    assert np.isfinite(y[[0, 2, 3]]).all()
    dx, _, dw = oracle.bwd(dy, x, rstd, w)
    assert np.isnan(dx[1]).all() and np.isnan(dx[2]).all()
    assert np.isfinite(dx[[0, 3]]).all()
    assert set(np.flatnonzero(np.isnan(dw))) == {3, 7}
    x[0, 5] = 0x7FC0   # NaN in x
    rstd, y = oracle.fwd(x, w, EPS)
    assert np.isnan(rstd[0]) and np.isnan(y[0]).all()
    _, _, dw = oracle.bwd(dy, x, rstd, w)
    assert np.isnan(dw).all()
