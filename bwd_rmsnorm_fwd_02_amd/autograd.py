"""torch.autograd wiring of the library's entry points.

Argument marshalling only: every forward and backward runs in the library's
HIP kernels (the functions of this package); nothing here computes. Tensors
are [..., H] with the row as the last dimension: x BF16, the weight BF16 or
FP32. The forward saves its rstd (and, for LayerNorm, its mean) and hands
it to the backward entry point, which takes the forward's row statistics.
dw (dgamma, dbeta) comes back in FP32; autograd rounds it to the
weight's dtype when the weight is BF16, so FP32 master weights keep all of
it. RMSNorm takes [T, H] and [T, heads, H] tensors through the strided
entry points as they are, per-head views of a wider buffer included (rows of
H contiguous elements, 16-byte aligned base and strides); other tensors, and
incoming gradients that do not fit (an expanded one, say), are copied to a
contiguous tensor first.

* rms_norm(x, w) -> y.
* rms_norm_residual(x, r, w) -> (y, h): h = BF16(x + r), the updated
  residual stream, and y = RMSNorm(h). Its backward takes the gradient of y
  and the gradient reaching h from later layers (the residual stream) and
  returns one combined gradient for both x and r
  (rmsnorm_residual_bwd with dres).
* layer_norm(x, gamma, beta=None) -> y.
* RMSNorm and LayerNorm modules holding the weight parameters.

deterministic=True (the default) gives bit-reproducible dw; False allows a
varying reduction order (the library currently runs the same fixed-order
kernels in both modes).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (layernorm_bwd, layernorm_fwd, rmsnorm_bwd_strided, rmsnorm_fwd_strided,
               rmsnorm_residual_bwd_strided, rmsnorm_residual_fwd_strided)

__all__ = ["rms_norm", "rms_norm_residual", "layer_norm", "RMSNorm", "LayerNorm"]


def _rows(t: torch.Tensor, H: int) -> torch.Tensor:
    """[..., H] as contiguous [rows, H] (a view when already contiguous)."""
    return t.contiguous().view(-1, H)


def _strided_ok(t: torch.Tensor) -> bool:
    """A [T, H] or [T, heads, H] tensor the strided entry points take as it
    is: rows of H contiguous elements, base and strides 16-byte aligned."""
    if t.dim() not in (2, 3) or t.stride(-1) != 1 or t.data_ptr() % 16:
        return False
    return all(s >= 0 and s % 8 == 0 for s in t.stride()[:-1])


def _fit(t: torch.Tensor, shape) -> torch.Tensor:
    """t as a tensor of `shape` ([T, H] or [T, heads, H]) that the strided
    entry points take: t itself (or a view of it) when it fits, else a copy."""
    v = t if tuple(t.shape) == tuple(shape) else t.reshape(shape)
    if _strided_ok(v):
        return v
    v = v.contiguous()
    return v if _strided_ok(v) else v.clone()


def _row_shape(x: torch.Tensor):
    """The view the entry points get: x's own [T, H] or [T, heads, H] shape
    (per-head views of a wider buffer pass as they are), else [rows, H]."""
    H = x.shape[-1]
    return tuple(x.shape) if x.dim() in (2, 3) else (x.numel() // H, H)


class _RMSNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, eps, deterministic):
        xs = _fit(x, _row_shape(x))
        y, rstd = rmsnorm_fwd_strided(xs, w, eps)
        ctx.save_for_backward(xs, rstd, w)
        ctx.deterministic = deterministic
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        xs, rstd, w = ctx.saved_tensors
        dx, dw = rmsnorm_bwd_strided(_fit(dy, xs.shape), xs, rstd, w,
                                     deterministic=ctx.deterministic)
        return dx.view(dy.shape), dw, None, None


class _RMSNormResidualFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, r, w, eps, deterministic):
        shape = _row_shape(x)
        h, y, rstd = rmsnorm_residual_fwd_strided(_fit(x, shape), _fit(r, shape), w, eps)
        ctx.save_for_backward(h, rstd, w)
        ctx.deterministic = deterministic
        ctx.shape = x.shape
        # an output nobody used gets no gradient (None), not a tensor of zeros
        ctx.set_materialize_grads(False)
        return y.view(x.shape), h.view(x.shape)

    @staticmethod
    def backward(ctx, dy, dh_out):
        h, rstd, w = ctx.saved_tensors
        dys = torch.zeros_like(h) if dy is None else _fit(dy, h.shape)
        dres = None if dh_out is None else _fit(dh_out, h.shape)
        dh, dw = rmsnorm_residual_bwd_strided(dys, h, rstd, w, dres=dres,
                                              deterministic=ctx.deterministic)
        dh = dh.view(ctx.shape)
        return dh, dh, dw, None, None


class _LayerNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, gamma, beta, eps, deterministic):
        H = x.shape[-1]
        x2 = _rows(x, H)
        y, mean, rstd = layernorm_fwd(x2, gamma, beta, eps)
        ctx.save_for_backward(x2, mean, rstd, gamma)
        ctx.deterministic = deterministic
        ctx.has_beta = beta is not None
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, mean, rstd, gamma = ctx.saved_tensors
        dx, dgamma, dbeta = layernorm_bwd(_rows(dy, x2.shape[1]), x2, mean, rstd, gamma,
                                          deterministic=ctx.deterministic)
        return dx.view(dy.shape), dgamma, (dbeta if ctx.has_beta else None), None, None


def rms_norm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
             deterministic: bool = True) -> torch.Tensor:
    """RMSNorm of x[..., H] (BF16) with weight w[H] (BF16 or FP32), differentiable."""
    return _RMSNormFn.apply(x, w, eps, deterministic)


def rms_norm_residual(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                      deterministic: bool = True):
    """(y, h) with h = BF16(x + r) and y = RMSNorm(h), differentiable in x, r and w."""
    return _RMSNormResidualFn.apply(x, r, w, eps, deterministic)


def layer_norm(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
               eps: float = 1e-5, deterministic: bool = True) -> torch.Tensor:
    """LayerNorm of x[..., H] (BF16) with gamma (and beta), differentiable."""
    return _LayerNormFn.apply(x, gamma, beta, eps, deterministic)


class RMSNorm(torch.nn.Module):
    """RMSNorm over the last dimension with a learnable weight (ones at start).
    forward(x) -> y; forward(x, residual) -> (y, h) with h = BF16(x + residual)."""

    def __init__(self, hidden: int, eps: float = 1e-6, weight_dtype: torch.dtype = torch.float32,
                 deterministic: bool = True, device=None):
        super().__init__()
        self.eps = eps
        self.deterministic = deterministic
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=weight_dtype, device=device))

    def forward(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None):
        if residual is None:
            return rms_norm(x, self.weight, self.eps, self.deterministic)
        return rms_norm_residual(x, residual, self.weight, self.eps, self.deterministic)


class LayerNorm(torch.nn.Module):
    """LayerNorm over the last dimension with learnable gamma (ones) and beta
    (zeros, or none with bias=False)."""

    def __init__(self, hidden: int, eps: float = 1e-5, bias: bool = True,
                 weight_dtype: torch.dtype = torch.float32, deterministic: bool = True,
                 device=None):
        super().__init__()
        self.eps = eps
        self.deterministic = deterministic
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=weight_dtype, device=device))
        self.bias = (torch.nn.Parameter(torch.zeros(hidden, dtype=weight_dtype, device=device))
                     if bias else None)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return layer_norm(x, self.weight, self.bias, self.eps, self.deterministic)
