"""RMSNorm for training on MI355X (gfx950): Python face of the C ABI.

The functions below carry the C ABI's names (include/rmsnorm.h) and only
marshal torch tensors into pointers, views and the current HIP stream; the
work is done by the HIP kernels in ``libbwd_rmsnorm.so``. Tensors must live
on a ROCm device. Outputs not supplied are allocated with torch.

Tensor conventions: x/dy/y/dx/h/r/dres are ``torch.bfloat16`` tensors of
shape [T, H] (plain) or [T, heads, H] (per-head view; any strides whose last
one is 1); w is bfloat16 or float32 of shape [H]; rstd is float32 of
[T] / [T, heads]; dw is float32 [H].
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import RMSNormError, View  # noqa: F401

__all__ = [
    "rmsnorm_fwd", "rmsnorm_fwd_strided", "rmsnorm_residual_fwd", "rmsnorm_residual_fwd_strided",
    "rmsnorm_bwd", "rmsnorm_bwd_strided", "rmsnorm_bwd_recompute", "rmsnorm_residual_bwd",
    "rmsnorm_residual_bwd_strided", "rmsnorm_bwd_strided_noalloc", "layernorm_fwd", "layernorm_bwd",
    "layernorm_bwd_workspace_bytes", "rmsnorm_bwd_workspace_bytes",
    "rmsnorm_workspace_init", "rmsnorm_status_string", "rmsnorm_route_query",
    "rmsnorm_route_override", "rmsnorm_timing_enable", "rmsnorm_timing_read",
    "RMSNormError", "View",
    "rms_norm", "rms_norm_residual", "layer_norm", "RMSNorm", "LayerNorm",
]


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[ctypes.c_void_p]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _wdtype(w: torch.Tensor) -> int:
    if w.dtype == torch.bfloat16:
        return _lib.RMSN_BF16
    if w.dtype == torch.float32:
        return _lib.RMSN_F32
    raise TypeError(f"weight dtype must be bfloat16 or float32, got {w.dtype}")


# ------------------------------------------------------- argument checks
#
# The C ABI takes raw pointers and trusts the shapes it is told: a tensor of
# the wrong dtype, length, device or layout would be read or written out of
# bounds on the GPU. Every tensor argument is therefore checked here before
# its pointer is taken; failures raise TypeError (type, dtype, device) or
# ValueError (shape, layout). Each tensor is checked for dtype, shape and
# layout first and for its device last, and every wrapper ends its checks
# with _need_gpu, so the host checks also run (and are tested) on tensors
# that live on the CPU.

def _on_device(name: str, t: torch.Tensor, dev: torch.device) -> None:
    if t.device != dev:
        raise TypeError(f"{name} is on {t.device}, expected {dev} (the device of the input)")


def _need_tensor(name: str, t) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")


def _need_gpu(dev: torch.device) -> None:
    if dev.type != "cuda":
        raise TypeError(f"the tensors must live on a ROCm device, not {dev}")


def _need_bf16(name: str, t: torch.Tensor, dev: Optional[torch.device] = None) -> None:
    _need_tensor(name, t)
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if dev is not None:
        _on_device(name, t, dev)


def _need_act(name: str, t: torch.Tensor, dev: torch.device, shape) -> None:
    """A contiguous BF16 activation of exactly `shape` on `dev`."""
    _need_bf16(name, t)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (use the *_strided entry points for views)")
    _on_device(name, t, dev)


def _need_f32(name: str, t: torch.Tensor, dev: torch.device, numel: int) -> None:
    """A contiguous float32 tensor of `numel` elements on `dev` (rstd, dw, ...)."""
    _need_tensor(name, t)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _on_device(name, t, dev)


def _need_weight(name: str, w: torch.Tensor, dev: torch.device, H: int) -> int:
    """A contiguous [H] bfloat16 or float32 weight on `dev`; returns its C dtype."""
    _need_tensor(name, w)
    wd = _wdtype(w)
    if tuple(w.shape) != (H,):
        raise ValueError(f"{name} has shape {tuple(w.shape)}, expected ({H},)")
    if not w.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _on_device(name, w, dev)
    return wd


def _ws_bytes(name: str, ws: Optional[torch.Tensor], dev: torch.device) -> int:
    if ws is None:
        return 0
    _need_tensor(name, ws)
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _on_device(name, ws, dev)
    return ws.numel() * ws.element_size()


def _view(t: torch.Tensor) -> View:
    """[T, H] or [T, heads, H] tensor -> C view (element strides)."""
    if t.dim() == 2:
        T, H = t.shape
        if t.stride(1) != 1:
            raise ValueError("the last dimension must be contiguous")
        return View(T, 1, H, t.stride(0), 0)
    if t.dim() == 3:
        T, heads, H = t.shape
        if t.stride(2) != 1:
            raise ValueError("the last dimension must be contiguous")
        return View(T, heads, H, t.stride(0), t.stride(1))
    raise ValueError("expected a [T, H] or [T, heads, H] tensor")


def _need_view(name: str, t: torch.Tensor, dev: torch.device, shape) -> View:
    """A BF16 [T, H] or [T, heads, H] view of exactly `shape` on `dev`."""
    _need_bf16(name, t)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    v = _view(t)
    _on_device(name, t, dev)
    return v


def _contig2d(name: str, t: torch.Tensor) -> Tuple[int, int]:
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [T, H] tensor")
    return t.shape[0], t.shape[1]


# ------------------------------------------------------------------ forward

def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                y: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None):
    """y, rstd = RMSNorm forward of contiguous x[T, H]."""
    _need_bf16("x", x)
    T, H = _contig2d("x", x)
    dev = x.device
    wd = _need_weight("w", w, dev, H)
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    _need_act("y", y, dev, (T, H))
    _need_f32("rstd", rstd, dev, T)
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_fwd(_ptr(x), _ptr(w), wd, float(eps), _ptr(y),
                                       _ptr(rstd), T, H, _stream(dev)))
    return y, rstd


def rmsnorm_fwd_strided(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                        y: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None):
    """Forward over a [T, heads, H] (or [T, H]) view with arbitrary row strides."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    wd = _need_weight("w", w, dev, xv.H)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    yv = _need_view("y", y, dev, x.shape)
    _need_f32("rstd", rstd, dev, xv.T * xv.heads)
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_fwd_strided(_ptr(x), xv, _ptr(w), wd, float(eps),
                                               _ptr(y), yv, _ptr(rstd), _stream(dev)))
    return y, rstd


def rmsnorm_residual_fwd(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                         h: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                         rstd: Optional[torch.Tensor] = None):
    """h = BF16(x + r); y, rstd = RMSNorm(h). Returns (h, y, rstd)."""
    _need_bf16("x", x)
    T, H = _contig2d("x", x)
    dev = x.device
    _need_act("r", r, dev, (T, H))
    wd = _need_weight("w", w, dev, H)
    h = torch.empty_like(x) if h is None else h
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    _need_act("h", h, dev, (T, H))
    _need_act("y", y, dev, (T, H))
    _need_f32("rstd", rstd, dev, T)
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_residual_fwd(_ptr(x), _ptr(r), _ptr(w), wd, float(eps),
                                                _ptr(h), _ptr(y), _ptr(rstd), T, H,
                                                _stream(dev)))
    return h, y, rstd


def rmsnorm_residual_fwd_strided(x: torch.Tensor, r: torch.Tensor, w: torch.Tensor,
                                 eps: float = 1e-6, h: Optional[torch.Tensor] = None,
                                 y: Optional[torch.Tensor] = None,
                                 rstd: Optional[torch.Tensor] = None):
    """The residual forward over [T, heads, H] (or [T, H]) views; each tensor
    keeps its own strides. Returns (h, y, rstd)."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    rv = _need_view("r", r, dev, x.shape)
    wd = _need_weight("w", w, dev, xv.H)
    if h is None:
        h = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    if rstd is None:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    hv = _need_view("h", h, dev, x.shape)
    yv = _need_view("y", y, dev, x.shape)
    _need_f32("rstd", rstd, dev, xv.T * xv.heads)
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_residual_fwd_strided(_ptr(x), xv, _ptr(r), rv, _ptr(w), wd,
                                                        float(eps), _ptr(h), hv, _ptr(y), yv,
                                                        _ptr(rstd), _stream(dev)))
    return h, y, rstd


# ----------------------------------------------------------------- backward

_WS_CACHE = {}


def rmsnorm_bwd_workspace_bytes(rows: int, H: int, w_dtype: torch.dtype, deterministic: bool) -> int:
    wd = _lib.RMSN_BF16 if w_dtype == torch.bfloat16 else _lib.RMSN_F32
    return int(_lib.load().rmsnorm_bwd_workspace_bytes(rows, H, wd, int(bool(deterministic))))


def rmsnorm_workspace_init(ws: torch.Tensor) -> None:
    _need_tensor("workspace", ws)
    nbytes = _ws_bytes("workspace", ws, ws.device)
    _need_gpu(ws.device)
    _lib.check(_lib.load().rmsnorm_workspace_init(_ptr(ws), nbytes, _stream(ws.device)))


def _workspace(dev: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    """Scratch workspace kept per (device, stream); the kernels need no
    initialisation of it."""
    if nbytes == 0:
        return None
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        raw = torch.empty(max(nbytes, 1 << 20) + 256, dtype=torch.uint8, device=dev)
        ws = raw[(-raw.data_ptr()) % 256:]
        _WS_CACHE[key] = ws
    return ws


def _bwd_outputs(dev, like_shape, H, dx, dw):
    if dx is None:
        dx = torch.empty(like_shape, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(H, dtype=torch.float32, device=dev) if dw is None else dw
    _need_f32("dw", dw, dev, H)
    return dx, dw


def rmsnorm_bwd(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor, w: torch.Tensor,
                deterministic: bool = True, dx: Optional[torch.Tensor] = None,
                dw: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """dx, dw of RMSNorm for contiguous [T, H] tensors."""
    _need_bf16("x", x)
    T, H = _contig2d("x", x)
    dev = x.device
    _need_act("dy", dy, dev, (T, H))
    _need_f32("rstd", rstd, dev, T)
    wd = _need_weight("w", w, dev, H)
    dx, dw = _bwd_outputs(dev, (T, H), H, dx, dw)
    _need_act("dx", dx, dev, (T, H))
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = rmsnorm_bwd_workspace_bytes(T, H, w.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(rstd), _ptr(w), wd,
                                       int(bool(deterministic)), _ptr(dx), _ptr(dw), T, H,
                                       _ptr(ws), nbytes, _stream(dev)))
    return dx, dw


def rmsnorm_bwd_strided(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor, w: torch.Tensor,
                        deterministic: bool = True, dx: Optional[torch.Tensor] = None,
                        dw: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Backward over [T, heads, H] views; dw sums over T and heads."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    rows = xv.T * xv.heads
    dyv = _need_view("dy", dy, dev, x.shape)
    _need_f32("rstd", rstd, dev, rows)
    wd = _need_weight("w", w, dev, xv.H)
    dx, dw = _bwd_outputs(dev, x.shape, xv.H, dx, dw)
    dxv = _need_view("dx", dx, dev, x.shape)
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = rmsnorm_bwd_workspace_bytes(rows, xv.H, w.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().rmsnorm_bwd_strided(_ptr(dy), dyv, _ptr(x), xv, _ptr(rstd),
                                               _ptr(w), wd, int(bool(deterministic)),
                                               _ptr(dx), dxv, _ptr(dw), _ptr(ws), nbytes,
                                               _stream(dev)))
    return dx, dw


def rmsnorm_bwd_strided_noalloc(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor,
                                w: torch.Tensor, deterministic: bool = True,
                                dx: Optional[torch.Tensor] = None,
                                dw: Optional[torch.Tensor] = None):
    """rmsnorm_bwd_strided with the library's fixed scratch as workspace (no
    allocation by the library; calls on one device must not overlap). Pass
    dx and dw to allocate nothing here either."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    rows = xv.T * xv.heads
    dyv = _need_view("dy", dy, dev, x.shape)
    _need_f32("rstd", rstd, dev, rows)
    wd = _need_weight("w", w, dev, xv.H)
    dx, dw = _bwd_outputs(dev, x.shape, xv.H, dx, dw)
    dxv = _need_view("dx", dx, dev, x.shape)
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_bwd_strided_noalloc(_ptr(dy), dyv, _ptr(x), xv, _ptr(rstd),
                                                       _ptr(w), wd, int(bool(deterministic)),
                                                       _ptr(dx), dxv, _ptr(dw), _stream(dev)))
    return dx, dw


def rmsnorm_bwd_recompute(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                          deterministic: bool = True, dx: Optional[torch.Tensor] = None,
                          dw: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """Backward without the forward's rstd (recomputed from x in the kernel),
    over [T, H] or [T, heads, H] views; dw sums over T and heads."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    rows = xv.T * xv.heads
    dyv = _need_view("dy", dy, dev, x.shape)
    wd = _need_weight("w", w, dev, xv.H)
    dx, dw = _bwd_outputs(dev, x.shape, xv.H, dx, dw)
    dxv = _need_view("dx", dx, dev, x.shape)
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = rmsnorm_bwd_workspace_bytes(rows, xv.H, w.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().rmsnorm_bwd_recompute(_ptr(dy), dyv, _ptr(x), xv, _ptr(w),
                                                 wd, float(eps), int(bool(deterministic)),
                                                 _ptr(dx), dxv, _ptr(dw), _ptr(ws), nbytes,
                                                 _stream(dev)))
    return dx, dw


def rmsnorm_residual_bwd(dy: torch.Tensor, h: torch.Tensor, rstd: torch.Tensor, w: torch.Tensor,
                         dres: Optional[torch.Tensor] = None, deterministic: bool = True,
                         dh: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """dh (the combined gradient for x and r) and dw of the residual form."""
    _need_bf16("h", h)
    T, H = _contig2d("h", h)
    dev = h.device
    _need_act("dy", dy, dev, (T, H))
    if dres is not None:
        _need_act("dres", dres, dev, (T, H))
    _need_f32("rstd", rstd, dev, T)
    wd = _need_weight("w", w, dev, H)
    dh, dw = _bwd_outputs(dev, (T, H), H, dh, dw)
    _need_act("dh", dh, dev, (T, H))
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = rmsnorm_bwd_workspace_bytes(T, H, w.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().rmsnorm_residual_bwd(_ptr(dy), _ptr(h), _ptr(dres), _ptr(rstd), _ptr(w),
                                                wd, int(bool(deterministic)), _ptr(dh),
                                                _ptr(dw), T, H, _ptr(ws), nbytes,
                                                _stream(dev)))
    return dh, dw


def rmsnorm_residual_bwd_strided(dy: torch.Tensor, h: torch.Tensor, rstd: torch.Tensor,
                                 w: torch.Tensor, dres: Optional[torch.Tensor] = None,
                                 deterministic: bool = True, dh: Optional[torch.Tensor] = None,
                                 dw: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None):
    """The residual backward over [T, heads, H] (or [T, H]) views; dw sums
    over T and heads. Returns (dh, dw)."""
    _need_bf16("h", h)
    dev = h.device
    hv = _view(h)
    rows = hv.T * hv.heads
    dyv = _need_view("dy", dy, dev, h.shape)
    dresv = _need_view("dres", dres, dev, h.shape) if dres is not None else View(0, 1, hv.H, 0, 0)
    _need_f32("rstd", rstd, dev, rows)
    wd = _need_weight("w", w, dev, hv.H)
    dh, dw = _bwd_outputs(dev, h.shape, hv.H, dh, dw)
    dhv = _need_view("dh", dh, dev, h.shape)
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = rmsnorm_bwd_workspace_bytes(rows, hv.H, w.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().rmsnorm_residual_bwd_strided(
        _ptr(dy), dyv, _ptr(h), hv, _ptr(dres), dresv, _ptr(rstd), _ptr(w), wd,
        int(bool(deterministic)), _ptr(dh), dhv, _ptr(dw), _ptr(ws), nbytes, _stream(dev)))
    return dh, dw


# ------------------------------------------------------- deferred dw reduce

def rmsnorm_bwd_partials_bytes(rows: int, H: int, w_dtype: torch.dtype) -> int:
    wd = _lib.RMSN_BF16 if w_dtype == torch.bfloat16 else _lib.RMSN_F32
    return int(_lib.load().rmsnorm_bwd_partials_bytes(rows, H, wd))


def _partials(dev, rows, H, w, partials):
    need = rmsnorm_bwd_partials_bytes(rows, H, w.dtype)
    if partials is None:
        raw = torch.empty(need + 256, dtype=torch.uint8, device=dev)
        partials = raw[(-raw.data_ptr()) % 256:]
    nbytes = _ws_bytes("partials", partials, dev)
    return partials, nbytes


def rmsnorm_bwd_strided_partials(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor,
                                 w: torch.Tensor, dx: Optional[torch.Tensor] = None,
                                 partials: Optional[torch.Tensor] = None):
    """The deterministic backward over views without its dw reduction: dx,
    and a uint8 buffer of dw partial rows for rmsnorm_dw_reduce_batch.
    Returns (dx, partials)."""
    _need_bf16("x", x)
    dev = x.device
    xv = _view(x)
    rows = xv.T * xv.heads
    dyv = _need_view("dy", dy, dev, x.shape)
    _need_f32("rstd", rstd, dev, rows)
    wd = _need_weight("w", w, dev, xv.H)
    if dx is None:
        dx = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    dxv = _need_view("dx", dx, dev, x.shape)
    if partials is not None:
        _ws_bytes("partials", partials, dev)
    _need_gpu(dev)
    partials, nbytes = _partials(dev, rows, xv.H, w, partials)
    _lib.check(_lib.load().rmsnorm_bwd_strided_partials(_ptr(dy), dyv, _ptr(x), xv, _ptr(rstd),
                                                        _ptr(w), wd, _ptr(dx), dxv, _ptr(partials),
                                                        nbytes, _stream(dev)))
    return dx, partials


def rmsnorm_residual_bwd_strided_partials(dy: torch.Tensor, h: torch.Tensor, rstd: torch.Tensor,
                                          w: torch.Tensor, dres: Optional[torch.Tensor] = None,
                                          dh: Optional[torch.Tensor] = None,
                                          partials: Optional[torch.Tensor] = None):
    """The residual form of rmsnorm_bwd_strided_partials. Returns (dh, partials)."""
    _need_bf16("h", h)
    dev = h.device
    hv = _view(h)
    rows = hv.T * hv.heads
    dyv = _need_view("dy", dy, dev, h.shape)
    dresv = _need_view("dres", dres, dev, h.shape) if dres is not None else View(0, 1, hv.H, 0, 0)
    _need_f32("rstd", rstd, dev, rows)
    wd = _need_weight("w", w, dev, hv.H)
    if dh is None:
        dh = torch.empty(h.shape, dtype=torch.bfloat16, device=dev)
    dhv = _need_view("dh", dh, dev, h.shape)
    if partials is not None:
        _ws_bytes("partials", partials, dev)
    _need_gpu(dev)
    partials, nbytes = _partials(dev, rows, hv.H, w, partials)
    _lib.check(_lib.load().rmsnorm_residual_bwd_strided_partials(
        _ptr(dy), dyv, _ptr(h), hv, _ptr(dres), dresv, _ptr(rstd), _ptr(w), wd, _ptr(dh), dhv,
        _ptr(partials), nbytes, _stream(dev)))
    return dh, partials


def rmsnorm_dw_reduce_batch(jobs) -> None:
    """Reduce the partial rows of earlier deferred backward calls into their
    dw, in one launch per 32 jobs of each partial precision. jobs: a list of
    (partials, rows, H, w_dtype, dw) with rows = T * heads of that call and
    dw an [H] FP32 tensor written in full."""
    n = len(jobs)
    arr = (_lib.DwJob * max(n, 1))()
    dev = None
    for i, (partials, rows, H, w_dtype, dw) in enumerate(jobs):
        _need_tensor("partials", partials)
        dev = partials.device if dev is None else dev
        nbytes = _ws_bytes("partials", partials, dev)
        _need_f32("dw", dw, dev, int(H))
        wd = _lib.RMSN_BF16 if w_dtype == torch.bfloat16 else _lib.RMSN_F32
        arr[i] = _lib.DwJob(partials.data_ptr(), nbytes, int(rows), int(H), wd, dw.data_ptr())
    if n == 0:
        return
    _need_gpu(dev)
    _lib.check(_lib.load().rmsnorm_dw_reduce_batch(arr, n, _stream(dev)))


# ---------------------------------------------------------------- LayerNorm

def layernorm_fwd(x: torch.Tensor, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
                  eps: float = 1e-5, y: Optional[torch.Tensor] = None,
                  mean: Optional[torch.Tensor] = None, rstd: Optional[torch.Tensor] = None):
    """y, mean, rstd = LayerNorm forward of contiguous x[T, H] (beta optional)."""
    _need_bf16("x", x)
    T, H = _contig2d("x", x)
    dev = x.device
    wd = _need_weight("gamma", gamma, dev, H)
    if beta is not None:
        _need_weight("beta", beta, dev, H)
        if beta.dtype != gamma.dtype:
            raise TypeError("gamma and beta must share one dtype")
    y = torch.empty_like(x) if y is None else y
    mean = torch.empty(T, dtype=torch.float32, device=dev) if mean is None else mean
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    _need_act("y", y, dev, (T, H))
    _need_f32("mean", mean, dev, T)
    _need_f32("rstd", rstd, dev, T)
    _need_gpu(dev)
    _lib.check(_lib.load().layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), wd,
                                         float(eps), _ptr(y), _ptr(mean), _ptr(rstd), T, H,
                                         _stream(dev)))
    return y, mean, rstd


def layernorm_bwd_workspace_bytes(rows: int, H: int, w_dtype: torch.dtype,
                                  deterministic: bool) -> int:
    wd = _lib.RMSN_BF16 if w_dtype == torch.bfloat16 else _lib.RMSN_F32
    return int(_lib.load().layernorm_bwd_workspace_bytes(rows, H, wd, int(bool(deterministic))))


def layernorm_bwd(dy: torch.Tensor, x: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor,
                  gamma: torch.Tensor, deterministic: bool = True,
                  dx: Optional[torch.Tensor] = None, dgamma: Optional[torch.Tensor] = None,
                  dbeta: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """dx, dgamma, dbeta of LayerNorm for contiguous [T, H] tensors."""
    _need_bf16("x", x)
    T, H = _contig2d("x", x)
    dev = x.device
    _need_act("dy", dy, dev, (T, H))
    _need_f32("mean", mean, dev, T)
    _need_f32("rstd", rstd, dev, T)
    wd = _need_weight("gamma", gamma, dev, H)
    dx = torch.empty_like(x) if dx is None else dx
    dgamma = torch.empty(H, dtype=torch.float32, device=dev) if dgamma is None else dgamma
    dbeta = torch.empty(H, dtype=torch.float32, device=dev) if dbeta is None else dbeta
    _need_act("dx", dx, dev, (T, H))
    _need_f32("dgamma", dgamma, dev, H)
    _need_f32("dbeta", dbeta, dev, H)
    _ws_bytes("workspace", workspace, dev)
    _need_gpu(dev)
    need = layernorm_bwd_workspace_bytes(T, H, gamma.dtype, deterministic)
    ws = workspace if workspace is not None else _workspace(dev, need)
    nbytes = _ws_bytes("workspace", ws, dev)
    _lib.check(_lib.load().layernorm_bwd(_ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd), _ptr(gamma),
                                         wd, int(bool(deterministic)), _ptr(dx),
                                         _ptr(dgamma), _ptr(dbeta), T, H, _ptr(ws), nbytes,
                                         _stream(dev)))
    return dx, dgamma, dbeta


# -------------------------------------------------------------- diagnostics

def rmsnorm_status_string(status: int) -> str:
    return _lib.status_string(status)


_OPS = {"fwd": 0, "bwd": 1, "ln_fwd": 2, "ln_bwd": 3}


def rmsnorm_route_query(op: str, rows: int, H: int, w_dtype: torch.dtype = torch.bfloat16,
                        deterministic: bool = True, residual: bool = False,
                        recompute: bool = False) -> dict:
    """Route-table entry for op 'fwd', 'bwd', 'ln_fwd' or 'ln_bwd' (host only,
    no GPU needed); the RMSNorm backward form is plain, residual or recompute."""
    info = _lib.RouteInfo()
    wd = _lib.RMSN_BF16 if w_dtype == torch.bfloat16 else _lib.RMSN_F32
    form = 2 if recompute else (1 if residual else 0)
    _lib.check(_lib.load().rmsnorm_route_query(_OPS[op], rows, H, wd,
                                               int(bool(deterministic)), form,
                                               ctypes.byref(info)))
    return info.as_dict()


def rmsnorm_route_override(op: str, **knobs) -> None:
    """Set (or, with no knobs, clear) the tuning override of op 'fwd', 'bwd',
    'ln_fwd' or 'ln_bwd'.
    Knobs: vec_per_lane, unroll, rows_per_block, blocks_per_cu, partial_f64
    (1 FP64, 2 FP32), kind (RMSN_KIND_BWD_ROW_DET/_ATOMIC, non-det only)."""
    o = _OPS[op]
    if not knobs:
        _lib.check(_lib.load().rmsnorm_route_override(o, None))
        return
    k = _lib.RouteKnobs(**knobs)
    _lib.check(_lib.load().rmsnorm_route_override(o, ctypes.byref(k)))


def rmsnorm_timing_enable(enable: bool = True) -> None:
    _lib.check(_lib.load().rmsnorm_timing_enable(int(bool(enable))))


def rmsnorm_timing_read() -> dict:
    """{timer index: (launches, total_ms)} accumulated since the last read."""
    n = _lib.RMSN_TIMER_COUNT
    launches = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    _lib.check(_lib.load().rmsnorm_timing_read(launches, ms, n))
    return {i: (int(launches[i]), float(ms[i])) for i in range(n)}


# torch.autograd wiring of the entry points above (marshalling only)
from .autograd import LayerNorm, RMSNorm, layer_norm, rms_norm, rms_norm_residual  # noqa: E402
