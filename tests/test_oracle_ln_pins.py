"""Pins for the LayerNorm part of the FP64 oracle (``oracle.ln_*``).

LayerNorm is the other normalisation of the same benchmark suite (ROCm
TransformerEngine PR "Microbenchmarking and CI performance regression test",
benchmark_normalization table). The oracle is checked against things other
than itself, chosen so that a plausible mistake (a dropped mean or c1 term,
a wrong sign, variance about zero instead of the mean, gamma applied after
beta, a missing rstd) fails at least one of them:

* central finite differences of L = sum(y * dy) with respect to x, gamma and
  beta, on small unrounded inputs;
* torch autograd through ``torch.nn.functional.layer_norm`` in float64 on
  the CPU (a library routine), and torch's biased variance and mean;
* closed forms: constant rows (xhat = 0, y = beta), H = 1, two-element rows;
* invariants: power-of-two scale invariance (bitwise, eps = 0), shift
  invariance, sum_j dx_j = 0 and sum_j dx_j xhat_j = rstd H c2 eps/(var+eps),
  linearity in dy;
* dbeta against math.fsum of dy, dgamma for T = 1 and against an exact
  rational sum.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import synth

EPS = 1e-5


def _loss(x, g, b, dy, eps):
    _, _, y = oracle.ln_fwd_f64(x, g, b, eps)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("T,H,eps", [(1, 2, 0.3), (2, 5, EPS), (3, 8, 0.05), (3, 7, 1e-3)])
def test_ln_backward_matches_finite_differences(T, H, eps):
    rng = np.random.default_rng(30 + H)
    x = rng.standard_normal((T, H)) + 0.5
    g = 1 + 0.3 * rng.standard_normal(H)
    b = 0.2 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    mu, rstd, _ = oracle.ln_fwd_f64(x, g, b, eps)
    dx, _, dg, db = oracle.ln_bwd_f64(dy, x, mu, rstd, g)
    h = 1e-5

    def fd(arr, f):
        out = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            out[idx] = (f(p) - f(m)) / (2 * h)
        return out

    fd_x = fd(x, lambda v: _loss(v, g, b, dy, eps))
    fd_g = fd(g, lambda v: _loss(x, v, b, dy, eps))
    fd_b = fd(b, lambda v: _loss(x, g, v, dy, eps))
    for got, ref in ((dx, fd_x), (dg, fd_g), (db, fd_b)):
        scale = np.max(np.abs(ref)) + 1e-30
        assert np.max(np.abs(got - ref)) / scale < 1e-7


@pytest.mark.parametrize("T,H,eps", [(4, 16, EPS), (7, 64, 0.01), (3, 256, 1e-6)])
def test_ln_matches_torch_layer_norm_autograd_float64(T, H, eps):
    rng = np.random.default_rng(40 + H)
    x = rng.standard_normal((T, H)) * 2.0 + 1.5
    g = 1 + 0.1 * rng.standard_normal(H)
    b = 0.1 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    yt = torch.nn.functional.layer_norm(xt, (H,), gt, bt, eps)
    yt.backward(torch.tensor(dy, dtype=torch.float64))
    mu, rstd, y = oracle.ln_fwd_f64(x, g, b, eps)
    var_t, mu_t = torch.var_mean(torch.tensor(x), dim=1, unbiased=False)
    np.testing.assert_allclose(mu, mu_t.numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(var_t.numpy() + eps), rtol=1e-13)
    dx, _, dg, db = oracle.ln_bwd_f64(dy, x, mu, rstd, g)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_ln_closed_form_rows():
    g = np.array([1.0, 2.0, -0.5, 3.0])
    b = np.array([0.25, -1.0, 0.5, 0.0])
    # constant row: mu = c, var = 0, rstd = 1/sqrt(eps), xhat = 0, y = beta
    mu, rstd, y = oracle.ln_fwd_f64(np.full((1, 4), 2.5), g, b, EPS)
    assert mu[0] == 2.5 and rstd[0] == 1.0 / math.sqrt(EPS) and np.array_equal(y[0], b)
    # its backward: dx = rstd (g*dy - mean(g*dy)), dgamma = 0, dbeta = dy
    dy = np.array([[1.0, -2.0, 0.5, 4.0]])
    dx, c, dg, db = oracle.ln_bwd_f64(dy, np.full((1, 4), 2.5), mu, rstd, g)
    gd = dy[0] * g
    np.testing.assert_allclose(dx[0], rstd[0] * (gd - gd.mean()), rtol=1e-15, atol=1e-15)
    assert np.all(dg == 0) and np.array_equal(db, dy[0]) and c[0, 1] == 0
    # two elements [a, b]: mu = (a+b)/2, var = ((a-b)/2)^2
    mu, rstd, y = oracle.ln_fwd_f64(np.array([[1.0, 4.0]]), np.ones(2), None, 0.75)
    assert mu[0] == 2.5 and rstd[0] == 1.0 / math.sqrt(2.25 + 0.75)
    assert y[0, 0] == -1.5 * rstd[0] and y[0, 1] == 1.5 * rstd[0]
    # H = 1: xhat = 0, y = beta, dx = 0
    mu, rstd, y = oracle.ln_fwd_f64(np.array([[-3.0]]), np.array([2.0]), np.array([0.5]), EPS)
    assert y[0, 0] == 0.5
    dx, _, _, _ = oracle.ln_bwd_f64(np.array([[7.0]]), np.array([[-3.0]]), mu, rstd, np.array([2.0]))
    assert dx[0, 0] == 0.0


def test_ln_power_of_two_scale_invariance_bitwise():
    wl = synth.make_ln(T=32, H=512, w_dtype="f32", seed=3, offset=1.0)
    x = oracle.bf16_to_double(wl.x)
    mu1, r1, y1 = oracle.ln_fwd_f64(x, wl.gamma.f64, wl.beta.f64, 0.0)
    mu4, r4, y4 = oracle.ln_fwd_f64(4.0 * x, wl.gamma.f64, wl.beta.f64, 0.0)
    assert np.array_equal(mu4, 4.0 * mu1) and np.array_equal(r4 * 4.0, r1)
    assert np.array_equal(y4, y1)


def test_ln_shift_invariance():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((8, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    b = 0.1 * rng.standard_normal(64)
    _, r1, y1 = oracle.ln_fwd_f64(x, g, b, EPS)
    mu2, r2, y2 = oracle.ln_fwd_f64(x + 37.0, g, b, EPS)
    np.testing.assert_allclose(mu2, np.mean(x, axis=1) + 37.0, rtol=1e-14)
    np.testing.assert_allclose(r2, r1, rtol=1e-12)
    np.testing.assert_allclose(y2, y1, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("eps", [0.0, 0.5])
def test_ln_dx_sums(eps):
    rng = np.random.default_rng(13)
    T, H = 16, 96
    x = rng.standard_normal((T, H)) + 2.0
    g = 1 + 0.1 * rng.standard_normal(H)
    dy = rng.standard_normal((T, H))
    mu, rstd, _ = oracle.ln_fwd_f64(x, g, None, eps)
    dx, c, _, _ = oracle.ln_bwd_f64(dy, x, mu, rstd, g)
    scale = np.sum(np.abs(dx), axis=1)
    assert np.all(np.abs(np.sum(dx, axis=1)) <= 1e-13 * scale)
    xhat = (x - mu[:, None]) * rstd[:, None]
    var = np.mean((x - mu[:, None]) ** 2, axis=1)
    expect = rstd * H * c[:, 1] * (eps / (var + eps))
    got = np.sum(dx * xhat, axis=1)
    scale2 = np.sum(np.abs(dx * xhat), axis=1)
    assert np.all(np.abs(got - expect) <= 1e-12 * scale2)
    if eps > 0:  # the eps term is not negligible on a typical row
        assert np.median(np.abs(expect) / scale2) > 1e-3


def test_ln_linear_in_dy():
    rng = np.random.default_rng(14)
    T, H = 9, 40
    x = rng.standard_normal((T, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    d1, d2 = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    mu, rstd, _ = oracle.ln_fwd_f64(x, g, None, EPS)
    a, b = 0.75, -2.5
    dxa, _, dga, dba = oracle.ln_bwd_f64(a * d1 + b * d2, x, mu, rstd, g)
    dx1, _, dg1, db1 = oracle.ln_bwd_f64(d1, x, mu, rstd, g)
    dx2, _, dg2, db2 = oracle.ln_bwd_f64(d2, x, mu, rstd, g)
    for u, v, w_ in ((dxa, dx1, dx2), (dga, dg1, dg2), (dba, db1, db2)):
        np.testing.assert_allclose(u, a * v + b * w_, rtol=1e-12, atol=1e-12)


def test_ln_dbeta_and_dgamma_sums():
    wl = synth.make_ln(T=3000, H=16, w_dtype="bf16", seed=15, offset=-2.0)
    mu, rstd, _ = oracle.ln_fwd(wl.x, wl.gamma.f64, wl.beta.f64, wl.eps, want_y=False)
    _, _, dg, db = oracle.ln_bwd(wl.dy, wl.x, mu, rstd, wl.gamma.f64, want_dx=False)
    dy = oracle.bf16_to_double(wl.dy)
    x = oracle.bf16_to_double(wl.x)
    for j in range(16):
        assert db[j] == math.fsum(dy[:, j])
    # dgamma against the exact rational sum of the FP64 terms dy * xhat
    u = 2.0 ** -53
    for j in range(0, 16, 5):
        terms = [Fraction(float(dy[t, j])) * Fraction(float((x[t, j] - mu[t]) * rstd[t]))
                 for t in range(3000)]
        exact = sum(terms, Fraction(0))
        mag = float(sum(abs(q) for q in terms))
        assert abs(float(Fraction(float(dg[j])) - exact)) <= 2.5 * u * mag + u * abs(float(exact))
    # T = 1: dgamma = dy * xhat exactly
    wl = synth.make_ln(T=1, H=64, w_dtype="f32", seed=16)
    mu, rstd, _ = oracle.ln_fwd(wl.x, wl.gamma.f64, wl.beta.f64, wl.eps, want_y=False)
    _, _, dg, db = oracle.ln_bwd(wl.dy, wl.x, mu, rstd, wl.gamma.f64)
    x = oracle.bf16_to_double(wl.x)[0]
    dy = oracle.bf16_to_double(wl.dy)[0]
    assert np.array_equal(dg, dy * ((x - mu[0]) * rstd[0])) and np.array_equal(db, dy)


def test_ln_bf16_and_f64_entry_points_agree():
    wl = synth.make_ln(T=20, H=48, w_dtype="bf16", seed=17, offset=3.0)
    m1, r1, y1 = oracle.ln_fwd(wl.x, wl.gamma.f64, wl.beta.f64, wl.eps)
    x = oracle.bf16_to_double(wl.x)
    m2, r2, y2 = oracle.ln_fwd_f64(x, wl.gamma.f64, wl.beta.f64, wl.eps)
    assert np.array_equal(m1, m2) and np.array_equal(r1, r2) and np.array_equal(y1, y2)
    a = oracle.ln_bwd(wl.dy, wl.x, m1, r1, wl.gamma.f64)
    b = oracle.ln_bwd_f64(oracle.bf16_to_double(wl.dy), x, m1, r1, wl.gamma.f64)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
