"""The torch.autograd wiring (bwd_rmsnorm_fwd_02_amd.autograd).

The wiring only marshals arguments, so every gradient it produces must have
exactly the bits of the direct entry-point calls on the same tensors:
rmsnorm_fwd / rmsnorm_bwd, rmsnorm_residual_fwd / rmsnorm_residual_bwd (the
gradient reaching h from later layers as dres, the combined gradient given
to both x and r), layernorm_fwd / layernorm_bwd. Checked with [..., H]
inputs of more than two dimensions, an expanded (stride 0) incoming
gradient, BF16 and FP32 weights (the BF16 weight's gradient is the FP32 dw
rounded by autograd), an unused residual output, LayerNorm with and without
beta, the modules, repeated backward passes (deterministic dw), per-head
views of a wider buffer (plain and residual; passed to the strided entry
points as they are) and a misaligned view (copied first). One case is also
held to the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
import oracle
from tests import synth
from tests.parity import check_dw, oracle_rstd32
from tests.test_parity_gpu import DEV, _announce, dev_bf16, dev_w

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b, what):
    a, b = a.detach(), b.detach()
    assert a.dtype == b.dtype and a.shape == b.shape, (what, a.dtype, b.dtype, a.shape, b.shape)
    assert torch.equal(_bits(a), _bits(b)), f"{what}: bits differ"


@pytest.mark.parametrize("shape,wdt", [((2, 1500, 1024), torch.float32),
                                       ((3000, 4096), torch.bfloat16),
                                       ((4, 8, 64, 256), torch.float32)])
def test_rms_norm_matches_entry_points(shape, wdt):
    _announce(f"autograd rms_norm {shape} {wdt}")
    H = shape[-1]
    g = torch.Generator(device="cpu").manual_seed(sum(shape))
    x = torch.randn(shape, generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(wdt).to(DEV).requires_grad_()
    dy = torch.randn(shape, generator=g).to(torch.bfloat16).to(DEV)
    y = rn.rms_norm(x, w, 1e-6)
    y.backward(dy)
    torch.cuda.synchronize()
    y_d, rstd = rn.rmsnorm_fwd(x.detach().view(-1, H), w.detach(), 1e-6)
    dx_d, dw_d = rn.rmsnorm_bwd(dy.view(-1, H), x.detach().view(-1, H), rstd, w.detach())
    torch.cuda.synchronize()
    _same(y.detach(), y_d.view(shape), "y")
    _same(x.grad, dx_d.view(shape), "dx")
    _same(w.grad, dw_d.to(wdt), "dw")
    # a second pass accumulates the same bits again (deterministic dw)
    g1 = w.grad.clone()
    w.grad = None
    rn.rms_norm(x, w, 1e-6).backward(dy)
    torch.cuda.synchronize()
    _same(w.grad, g1, "dw, second pass")


def test_rms_norm_expanded_gradient_and_oracle():
    """loss = y.sum(): the incoming gradient is an expanded tensor of ones."""
    T, H = 5000, 2048
    _announce(f"autograd rms_norm y.sum() T={T} H={H}")
    wl = synth.make(T=T, H=H, w_dtype="f32", seed=11)
    x = dev_bf16(wl.x).requires_grad_()
    w = dev_w(wl.w).requires_grad_()
    rn.rms_norm(x, w, wl.eps).sum().backward()
    torch.cuda.synchronize()
    ones = torch.ones(T, H, dtype=torch.bfloat16, device=DEV)
    _, rstd = rn.rmsnorm_fwd(x.detach(), w.detach(), wl.eps)
    dx_d, dw_d = rn.rmsnorm_bwd(ones, x.detach(), rstd, w.detach())
    torch.cuda.synchronize()
    _same(x.grad, dx_d, "dx")
    _same(w.grad, dw_d, "dw")
    _, r32 = oracle_rstd32(wl.x, wl.w.f64, wl.eps)
    dy1 = np.full(wl.x.shape, 0x3F80, dtype=wl.x.dtype)  # BF16 1.0
    _, _, dw64 = oracle.bwd(dy1, wl.x, r32.astype(np.float64), wl.w.f64, want_dx=False)
    check_dw("dw (oracle, dy = 1)", w.grad.cpu().numpy(), dw64)


@pytest.mark.parametrize("use_h", [True, False])
def test_rms_norm_residual_matches_entry_points(use_h):
    T, H = 3000, 1536
    _announce(f"autograd rms_norm_residual T={T} H={H} use_h={use_h}")
    g = torch.Generator(device="cpu").manual_seed(7)
    mk = lambda: torch.randn(2, T // 2, H, generator=g).to(torch.bfloat16).to(DEV)
    x, r = mk().requires_grad_(), mk().requires_grad_()
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(DEV).requires_grad_()
    a, b = mk(), mk()
    y, h = rn.rms_norm_residual(x, r, w, 1e-6)
    loss = (y.float() * a.float()).sum()
    if use_h:
        loss = loss + (h.float() * b.float()).sum()
    loss.backward()
    torch.cuda.synchronize()
    h_d, y_d, rstd = rn.rmsnorm_residual_fwd(x.detach().view(T, H), r.detach().view(T, H),
                                             w.detach(), 1e-6)
    # the incoming gradients: d loss / d y = a and d loss / d h = b, exactly
    dy = a.view(T, H)
    dres = b.view(T, H) if use_h else None
    dh_d, dw_d = rn.rmsnorm_residual_bwd(dy, h_d, rstd, w.detach(), dres=dres)
    torch.cuda.synchronize()
    _same(y.detach().view(T, H), y_d, "y")
    _same(h.detach().view(T, H), h_d, "h")
    _same(x.grad.view(T, H), dh_d, "dx")
    _same(r.grad.view(T, H), dh_d, "dr")
    _same(w.grad, dw_d, "dw")


@pytest.mark.parametrize("with_beta", [True, False])
def test_layer_norm_matches_entry_points(with_beta):
    T, H = 4096, 3584
    _announce(f"autograd layer_norm T={T} H={H} beta={with_beta}")
    g = torch.Generator(device="cpu").manual_seed(3)
    x = (torch.randn(T, H, generator=g) + 2.0).to(torch.bfloat16).to(DEV).requires_grad_()
    gamma = (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16).to(DEV).requires_grad_()
    beta = ((0.1 * torch.randn(H, generator=g)).to(torch.bfloat16).to(DEV).requires_grad_()
            if with_beta else None)
    dy = torch.randn(T, H, generator=g).to(torch.bfloat16).to(DEV)
    y = rn.layer_norm(x, gamma, beta, 1e-5)
    y.backward(dy)
    torch.cuda.synchronize()
    bd = beta.detach() if with_beta else None
    y_d, mean, rstd = rn.layernorm_fwd(x.detach(), gamma.detach(), bd, 1e-5)
    dx_d, dg_d, db_d = rn.layernorm_bwd(dy, x.detach(), mean, rstd, gamma.detach())
    torch.cuda.synchronize()
    _same(y.detach(), y_d, "y")
    _same(x.grad, dx_d, "dx")
    _same(gamma.grad, dg_d.to(torch.bfloat16), "dgamma")
    if with_beta:
        _same(beta.grad, db_d.to(torch.bfloat16), "dbeta")


def test_modules():
    T, H = 1024, 512
    _announce("autograd modules")
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(DEV)
    res = torch.randn(T, H, generator=g).to(torch.bfloat16).to(DEV)
    m = rn.RMSNorm(H, device=DEV)
    with torch.no_grad():
        m.weight.copy_(1 + 0.1 * torch.randn(H, generator=g))
    _same(m(x), rn.rms_norm(x, m.weight), "RMSNorm(x)")
    y, h = m(x, res)
    h_d, y_d, _ = rn.rmsnorm_residual_fwd(x, res, m.weight.detach())
    _same(y, y_d, "RMSNorm(x, residual) y")
    _same(h, h_d, "RMSNorm(x, residual) h")
    ln = rn.LayerNorm(H, weight_dtype=torch.bfloat16, device=DEV)
    _same(ln(x), rn.layer_norm(x, ln.weight, ln.bias), "LayerNorm(x)")
    ln(x).float().sum().backward()
    assert ln.weight.grad is not None and ln.bias.grad is not None
    assert ln.weight.grad.dtype == torch.bfloat16
    torch.cuda.synchronize()


def test_rms_norm_head_views():
    """Per-head views of a wider buffer go to the strided entry points as
    they are; the gradient lands in the view's columns of the buffer only."""
    T, heads, H, row = 2048, 24, 256, 8192
    _announce(f"autograd rms_norm head views T={T} heads={heads} H={H} row={row}")
    g = torch.Generator(device="cpu").manual_seed(9)
    buf = torch.randn(T, row, generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(DEV).requires_grad_()
    dy = torch.randn(T, heads, H, generator=g).to(torch.bfloat16).to(DEV)
    x = buf[:, : heads * H].view(T, heads, H)
    assert not x.is_contiguous()
    y = rn.rms_norm(x, w)
    y.backward(dy)
    torch.cuda.synchronize()
    xd = buf.detach()[:, : heads * H].view(T, heads, H)
    y_d, rstd = rn.rmsnorm_fwd_strided(xd, w.detach())
    dx_d, dw_d = rn.rmsnorm_bwd_strided(dy, xd, rstd, w.detach())
    torch.cuda.synchronize()
    _same(y, y_d, "y")
    _same(buf.grad[:, : heads * H].reshape(T, heads, H), dx_d, "dx")
    assert not torch.any(buf.grad[:, heads * H:]), "gradient outside the view"
    _same(w.grad, dw_d, "dw")


def test_rms_norm_residual_head_views():
    T, heads, H, row = 1024, 8, 256, 8192
    _announce(f"autograd rms_norm_residual head views T={T} heads={heads} H={H}")
    g = torch.Generator(device="cpu").manual_seed(10)
    bx = torch.randn(T, row, generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    br = torch.randn(T, row, generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16).to(DEV).requires_grad_()
    a = torch.randn(T, heads, H, generator=g).to(torch.bfloat16).to(DEV)
    b = torch.randn(T, heads, H, generator=g).to(torch.bfloat16).to(DEV)
    x = bx[:, : heads * H].view(T, heads, H)
    r = br[:, 2048: 2048 + heads * H].view(T, heads, H)
    y, h = rn.rms_norm_residual(x, r, w)
    ((y.float() * a.float()).sum() + (h.float() * b.float()).sum()).backward()
    torch.cuda.synchronize()
    xd = bx.detach()[:, : heads * H].view(T, heads, H)
    rd = br.detach()[:, 2048: 2048 + heads * H].view(T, heads, H)
    h_d, y_d, rstd = rn.rmsnorm_residual_fwd_strided(xd, rd, w.detach())
    dh_d, dw_d = rn.rmsnorm_residual_bwd_strided(a, h_d, rstd, w.detach(), dres=b)
    torch.cuda.synchronize()
    _same(y, y_d, "y")
    _same(h, h_d, "h")
    _same(bx.grad[:, : heads * H].reshape(T, heads, H), dh_d, "dx")
    _same(br.grad[:, 2048: 2048 + heads * H].reshape(T, heads, H), dh_d, "dr")
    _same(w.grad, dw_d.to(torch.bfloat16), "dw")


def test_rms_norm_misaligned_view_is_copied():
    """A view whose base is not 16-byte aligned is copied first: same bits
    as the direct call on the contiguous copy."""
    T, H = 777, 512
    _announce(f"autograd rms_norm misaligned view T={T} H={H}")
    g = torch.Generator(device="cpu").manual_seed(12)
    buf = torch.randn(T, H + 4, generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(DEV).requires_grad_()
    dy = torch.randn(T, H, generator=g).to(torch.bfloat16).to(DEV)
    x = buf[:, 4:]
    assert x.data_ptr() % 16 != 0
    y = rn.rms_norm(x, w)
    y.backward(dy)
    torch.cuda.synchronize()
    xc = x.detach().contiguous()
    y_d, rstd = rn.rmsnorm_fwd(xc, w.detach())
    dx_d, dw_d = rn.rmsnorm_bwd(dy, xc, rstd, w.detach())
    torch.cuda.synchronize()
    _same(y, y_d, "y")
    _same(buf.grad[:, 4:], dx_d, "dx")
    assert not torch.any(buf.grad[:, :4])
    _same(w.grad, dw_d, "dw")
