"""Seeded synthetic inputs for RMSNorm training workloads.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic; the HIP path and the oracle both take their inputs from
here.

Recipe (the pages' workloads are synthetic: flashinfer PR "fix(cake_rmsnorm):
sm_100a and sm_107a dw-accuracy backward routes", "Workload" paragraph):

* generator: ``numpy.random.default_rng(seed)`` (PCG64);
* activations x, r, dy, dres: ``standard_normal`` drawn in float32, rounded
  to BF16 with round-to-nearest-even (torch's conversion);
* weight: ``1 + 0.1 * standard_normal`` in float32, then rounded to the
  weight dtype (BF16 or left in FP32);
* heavy rows (large-T dw stress): ``round(0.01 * T)`` distinct rows chosen by
  ``rng.choice(T, k, replace=False)`` have x scaled by 8 (exact in BF16);
* per-head strided form: the whole ``[T, 8192]`` buffer is N(0,1); x is its
  ``[:, :24*256]`` columns seen as ``[T, 24, 256]`` (row stride 8192, head
  stride 256).

Draw order within a workload is fixed: weight, x (or the strided buffer),
heavy-row choice, r, dy, dres.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

EPS = 1e-6  # "Workload": eps 1e-6


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16), nearest-even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclasses.dataclass
class Weight:
    dtype: str            # "bf16" or "f32"
    bits: Optional[np.ndarray]   # uint16 patterns when dtype == "bf16"
    f32: np.ndarray       # the weight's values as float32 (exact)

    @property
    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def raw(self) -> np.ndarray:
        """The array handed to the library: uint16 bits or float32 values."""
        return self.bits if self.dtype == "bf16" else self.f32


def weight(rng: np.random.Generator, H: int, dtype: str) -> Weight:
    w32 = (1.0 + 0.1 * rng.standard_normal(H, dtype=np.float32)).astype(np.float32)
    if dtype == "bf16":
        b = bf16_bits(w32)
        return Weight("bf16", b, bits_to_f32(b))
    if dtype == "f32":
        return Weight("f32", None, w32)
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    """One seeded problem. Arrays are BF16 bit patterns unless noted.

    ``x``/``dy``/``r``/``dres`` are logical ``[rows, H]`` arrays (rows = T*heads,
    row = t*heads + head). For the strided per-head form, ``xbuf`` holds the
    whole ``[T, row_stride]`` buffer and ``x`` is the gathered view.
    """
    name: str
    T: int
    heads: int
    H: int
    w: Weight
    x: np.ndarray
    dy: np.ndarray
    r: Optional[np.ndarray] = None
    dres: Optional[np.ndarray] = None
    xbuf: Optional[np.ndarray] = None
    x_stride_t: int = 0
    x_stride_h: int = 0
    heavy_rows: Optional[np.ndarray] = None
    eps: float = EPS

    @property
    def rows(self) -> int:
        return self.T * self.heads


def make(T: int, H: int, w_dtype: str, seed: int, *, heads: int = 1,
         residual: bool = False, with_dres: bool = True, heavy_frac: float = 0.0,
         strided_row: int = 0, same_sign: bool = False, name: str = "") -> Workload:
    """Build a workload. ``strided_row`` > 0 selects the strided per-head form:
    x lives in a ``[T, strided_row]`` buffer with head stride H. ``same_sign``
    takes |x| and |dy| (every dy*xhat term positive, so dw grows like T)."""
    rng = np.random.default_rng(seed)
    w = weight(rng, H, w_dtype)
    rows = T * heads
    xbuf = None
    st_t, st_h = heads * H, H
    if strided_row:
        assert strided_row >= heads * H
        xbuf = normal_bf16(rng, (T, strided_row))
        x = np.ascontiguousarray(xbuf[:, : heads * H]).reshape(rows, H)
        st_t = strided_row
    else:
        x = normal_bf16(rng, (rows, H))
    heavy = None
    if heavy_frac > 0:
        k = int(round(heavy_frac * T))
        heavy = np.sort(rng.choice(T, k, replace=False))
        xf = bits_to_f32(x)
        xf[heavy] *= 8.0
        x = bf16_bits(xf)
    r = normal_bf16(rng, (rows, H)) if residual else None
    dy = normal_bf16(rng, (rows, H))
    if same_sign:
        x = x & np.uint16(0x7FFF)   # clear the BF16 sign bit: |x|
        dy = dy & np.uint16(0x7FFF)
    dres = normal_bf16(rng, (rows, H)) if (residual and with_dres) else None
    return Workload(name=name, T=T, heads=heads, H=H, w=w, x=x, dy=dy, r=r,
                    dres=dres, xbuf=xbuf, x_stride_t=st_t, x_stride_h=st_h,
                    heavy_rows=heavy)


# Input families for accuracy sweeps (the pages use three families; their
# definitions are not given, so these are this library's choice).
FAMILIES = {
    "normal": dict(),
    "heavy_rows": dict(heavy_frac=0.01),
    "same_sign": dict(same_sign=True),
}

# The five workloads the method is quoted on (T, H, weight dtype, form).
CONFIGS = {
    "c1_T64_H256_f32w": dict(T=64, H=256, w_dtype="f32"),
    "c2_T4096_H4096_bf16w": dict(T=4096, H=4096, w_dtype="bf16"),
    "c3_T131072_H2048_f32w_heavy": dict(T=131072, H=2048, w_dtype="f32", heavy_frac=0.01),
    "c4_res_T16384_H6144_bf16w": dict(T=16384, H=6144, w_dtype="bf16", residual=True),
    "c5a_heads_T32768x24x256_strided8192_f32w": dict(T=32768, heads=24, H=256, w_dtype="f32",
                                                     strided_row=8192),
    "c5b_heads_T32768x4x256_f32w": dict(T=32768, heads=4, H=256, w_dtype="f32"),
}


# The other widths of the pages' seven (256, 512, 1536, 2048, 4096, 5120,
# 6144), at large token counts (their top windows run up to T 1,048,576).
WIDTH_CONFIGS = {
    "w512_T1048576_bf16w": dict(T=1048576, H=512, w_dtype="bf16"),
    "w1536_T262144_f32w": dict(T=262144, H=1536, w_dtype="f32"),
    "w5120_T65536_bf16w": dict(T=65536, H=5120, w_dtype="bf16"),
    # the widest shape of the TE page's normalization table (8192 x 16384)
    "w16384_T8192_bf16w": dict(T=8192, H=16384, w_dtype="bf16"),
}


def config(name: str, seed: int = 0, **overrides) -> Workload:
    kw = dict(CONFIGS[name] if name in CONFIGS else WIDTH_CONFIGS[name])
    kw.update(overrides)
    return make(seed=seed, name=name, **kw)


# ------------------------------------------------------------------ LayerNorm

@dataclasses.dataclass
class LNWorkload:
    """One seeded LayerNorm problem: x, dy BF16 bits [T, H]; gamma, beta in
    the weight dtype."""
    name: str
    T: int
    H: int
    gamma: Weight
    beta: Weight
    x: np.ndarray
    dy: np.ndarray
    eps: float = 1e-5


def make_ln(T: int, H: int, w_dtype: str, seed: int, *, offset: float = 0.0,
            name: str = "") -> LNWorkload:
    """x = N(0,1) + offset and dy = N(0,1), drawn in float32 and rounded to
    BF16; gamma = 1 + 0.1 N(0,1) and beta = 0.1 N(0,1) in the weight dtype.
    Draw order: gamma, beta, x, dy. A nonzero offset stresses the mean
    subtraction (|mu| well above the spread of a row)."""
    rng = np.random.default_rng(seed)
    gamma = weight(rng, H, w_dtype)
    b32 = (0.1 * rng.standard_normal(H, dtype=np.float32)).astype(np.float32)
    if w_dtype == "bf16":
        bb = bf16_bits(b32)
        beta = Weight("bf16", bb, bits_to_f32(bb))
    else:
        beta = Weight("f32", None, b32)
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32) + np.float32(offset))
    dy = normal_bf16(rng, (T, H))
    return LNWorkload(name=name, T=T, H=H, gamma=gamma, beta=beta, x=x, dy=dy)


# LayerNorm workloads: the shapes of the benchmark_normalization table of
# ROCm TransformerEngine PR "Microbenchmarking and CI performance regression
# test" (M tokens x hidden, BF16), largest M.
LN_CONFIGS = {
    "ln_T8192_H4096_bf16w": dict(T=8192, H=4096, w_dtype="bf16"),
    "ln_T8192_H8192_bf16w": dict(T=8192, H=8192, w_dtype="bf16"),
    "ln_T8192_H3584_bf16w": dict(T=8192, H=3584, w_dtype="bf16"),
    "ln_T8192_H16384_bf16w": dict(T=8192, H=16384, w_dtype="bf16"),
}


def ln_config(name: str, seed: int = 0, **overrides) -> LNWorkload:
    kw = dict(LN_CONFIGS[name])
    kw.update(overrides)
    return make_ln(seed=seed, name=name, **kw)
