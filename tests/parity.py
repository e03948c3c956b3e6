"""Tolerances and comparisons between the HIP path and the FP64 oracle.

Budgets (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
backward routes"):
* dw: per element |dw - dw64| <= 1e-4 + 1e-4 |dw64| (the dw budget of
  "Changed windows by reason": absolute and relative tolerance 1e-4 on each
  element against FP64), checked against the oracle's sum taken at the FP32
  rstd the backward is given and against its sum at the rstd recomputed in
  FP64 (the page's two rstd forms);
* y and dx: within one BF16 ulp of the FP64 value rounded to BF16. y is
  checked strictly. dx = rstd*(g - xhat*c) can cancel, and no FP32 evaluation
  can promise one ulp there: an element whose FP32 evaluation bound E exceeds
  half a BF16 ulp of the FP64 value passes if |dx - dx64| <= ulp + E; such
  elements are counted and reported;
* rstd: relative 1e-6 against the FP64 value;
* h = BF16(x + r): bit-exact; deterministic dw: bit-identical run to run.
"""
from __future__ import annotations

import math

import numpy as np

from tests import synth
import oracle

DW_ATOL = 1e-4
DW_RTOL = 1e-4
RSTD_RTOL = 1e-6
U32 = 2.0 ** -24


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """ULP of BF16 at the magnitude of v (float64): 2^(e - 7) for the binade
    exponent e = floor(log2 |v|), read from the float64 exponent field (exact,
    unlike a rounded log2 at the top of a binade); 2^-133 below the normal
    range and at zero."""
    a = np.abs(np.asarray(v, np.float64))
    e = ((a.view(np.int64) >> 52) & 0x7FF) - 1023
    e = np.maximum(e, -126)
    u = ((e + (1023 - 7)) << 52).view(np.float64)
    return np.where(a > 0, u, 2.0 ** -133)


def to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def check_bf16_strict(name: str, got_bits: np.ndarray, ref64: np.ndarray) -> None:
    got = to_f64(got_bits)
    ulp = bf16_ulp(ref64)
    err = np.abs(got - ref64)
    bad = err > ulp
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{name}: {int(bad.sum())} elements beyond 1 BF16 ulp; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref64[tuple(i)]!r}")


def dx_bound(x64, dy64, w64, rstd, c, H, dres64=None):
    """FP32 evaluation bound E for dx = rstd*(dy*w - x*rstd*c) (+ dres)."""
    g = np.abs(dy64 * w64[None, :])
    xh = np.abs(x64 * rstd[:, None])
    sgx = np.sum(g * xh, axis=1) / H  # (1/H) sum |g*xhat|
    gamma_c = (math.log2(max(H, 2)) + 16.0) * U32
    E = rstd[:, None] * (4 * U32 * (g + xh * np.abs(c)[:, None]) + xh * gamma_c * sgx[:, None])
    if dres64 is not None:
        E = E + 2 * U32 * np.abs(dres64)
    return E


def check_dx(name: str, got_bits: np.ndarray, dx64: np.ndarray, E: np.ndarray) -> int:
    """Returns the number of exempted (cancellation) elements."""
    got = to_f64(got_bits)
    ulp = bf16_ulp(dx64)
    err = np.abs(got - dx64)
    strict = err <= ulp
    exempt = (~strict) & (E > 0.5 * ulp)
    ok = strict | (exempt & (err <= ulp + E))
    if not np.all(ok):
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{name}: {int((~ok).sum())} elements out of tolerance; first at {i}: "
                             f"got {got[i]!r} ref {dx64[i]!r} ulp {ulp[i]!r} E {E[i]!r}")
    return int(exempt.sum())


def check_dw(name: str, dw_gpu: np.ndarray, dw64: np.ndarray) -> float:
    """Returns the worst error as a fraction of the budget."""
    dw_gpu = np.asarray(dw_gpu, np.float64)
    tol = DW_ATOL + DW_RTOL * np.abs(dw64)
    frac = np.abs(dw_gpu - dw64) / tol
    worst = float(np.max(frac)) if frac.size else 0.0
    if not worst <= 1.0:
        j = int(np.argmax(frac))
        raise AssertionError(f"{name}: dw error {worst:.3f} of budget at column {j}: "
                             f"got {dw_gpu[j]!r} ref {dw64[j]!r}")
    return worst


def check_rstd(name: str, got: np.ndarray, ref64: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    rel = np.abs(got - ref64) / np.abs(ref64)
    worst = float(np.max(rel)) if rel.size else 0.0
    if not worst <= RSTD_RTOL:
        i = int(np.argmax(rel))
        raise AssertionError(f"{name}: rstd relative error {worst:.3e} at row {i}")
    return worst


def oracle_rstd32(x_bits: np.ndarray, w64: np.ndarray, eps: float):
    """The oracle's rstd in FP64 and rounded to FP32 (the backward's input)."""
    r64, _ = oracle.fwd(x_bits, w64, eps, want_y=False)
    return r64, oracle.round_f32(r64)


# ------------------------------------------------------------------ LayerNorm
#
# The same budgets for LayerNorm (the adjacent normalisation of ROCm
# TransformerEngine PR "Microbenchmarking and CI performance regression
# test", benchmark_normalization): dgamma and dbeta per element as dw; y and
# dx within one BF16 ulp of the FP64 value rounded to BF16, with the same
# cancellation exemption (y = xhat*gamma + beta can cancel too, so y gets a
# bound as well); mean and rstd within relative 1e-6 (the mean relative to
# the row's scale sqrt(mean^2 + var), since it can be near zero).

def ln_y_bound(x64, mu64, rstd64, gamma64, beta64):
    """FP32 evaluation bound for y = (x - mean)*rstd*gamma + beta, from a
    forward whose mean and rstd carry their own FP32 rounding."""
    xhat = (x64 - mu64[:, None]) * rstd64[:, None]
    scale = rstd64[:, None] * (np.abs(x64) + np.abs(mu64)[:, None])
    b = 0.0 if beta64 is None else np.abs(beta64)[None, :]
    return U32 * (4 * scale * np.abs(gamma64)[None, :] + 4 * np.abs(xhat * gamma64[None, :]) + 2 * b)


def ln_dx_bound(x64, dy64, gamma64, mu, rstd, c, H):
    """FP32 evaluation bound for dx = rstd*(g - c1 - xhat*c2) at the given
    (FP32) mean and rstd; c = [c1, c2] per row."""
    g = np.abs(dy64 * gamma64[None, :])
    xh = np.abs((x64 - mu[:, None]) * rstd[:, None])
    c1 = np.abs(c[:, 0])[:, None]
    c2 = np.abs(c[:, 1])[:, None]
    mg = np.mean(g, axis=1)[:, None]
    mgx = np.mean(g * xh, axis=1)[:, None]
    gamma_c = (math.log2(max(H, 2)) + 16.0) * U32
    return rstd[:, None] * (4 * U32 * (g + c1 + xh * c2) + 2 * U32 * xh * c2
                            + gamma_c * (mg + xh * mgx))


def check_ln_stats(name: str, mean_gpu, rstd_gpu, mu64, rstd64, var64) -> None:
    mean_gpu = np.asarray(mean_gpu, np.float64)
    scale = np.sqrt(mu64 * mu64 + var64)
    bad = np.abs(mean_gpu - mu64) > RSTD_RTOL * scale
    if np.any(bad):
        i = int(np.argmax(bad))
        raise AssertionError(f"{name}: mean off at row {i}: {mean_gpu[i]!r} vs {mu64[i]!r}")
    check_rstd(name + " rstd", rstd_gpu, rstd64)
