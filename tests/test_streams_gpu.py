"""Calls on several HIP streams at once.

Every entry point is asynchronous on the stream it is given, and two calls
may run concurrently when each has its own workspace (the Python binding
keeps one per device and stream). Here different problems run interleaved
on two streams (default priority), and every output must be bit for bit
what the same calls give one after another on the current stream: the
kernels share no state between calls, and the deterministic dw does not
depend on what else runs on the device.
"""
from __future__ import annotations

import pytest
import torch

import bwd_rmsnorm_fwd_02_amd as rn
from tests import synth
from tests.test_parity_gpu import DEV, _announce, dev_bf16, dev_w

pytestmark = pytest.mark.gpu


def _rms_problem(T, H, wdt, seed):
    wl = synth.make(T=T, H=H, w_dtype=wdt, seed=seed)
    return dict(x=dev_bf16(wl.x), dy=dev_bf16(wl.dy), w=dev_w(wl.w), eps=wl.eps)


def _ln_problem(T, H, seed):
    wl = synth.make_ln(T=T, H=H, w_dtype="bf16", seed=seed)
    return dict(x=dev_bf16(wl.x), dy=dev_bf16(wl.dy), g=dev_w(wl.gamma), b=dev_w(wl.beta), eps=wl.eps)


def _run_rms(p):
    y, rstd = rn.rmsnorm_fwd(p["x"], p["w"], p["eps"])
    dx, dw = rn.rmsnorm_bwd(p["dy"], p["x"], rstd, p["w"], deterministic=True)
    return [y, rstd, dx, dw]


def _run_ln(p):
    y, mean, rstd = rn.layernorm_fwd(p["x"], p["g"], p["b"], p["eps"])
    dx, dg, db = rn.layernorm_bwd(p["dy"], p["x"], mean, rstd, p["g"], deterministic=True)
    return [y, mean, rstd, dx, dg, db]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_two_streams_interleaved_match_sequential():
    _announce("two streams: RMSNorm 4096x4096 | RMSNorm 20000x256 + LayerNorm 2048x3584")
    a = _rms_problem(4096, 4096, "bf16", 101)
    b = _rms_problem(20000, 256, "f32", 102)
    c = _ln_problem(2048, 3584, 103)
    ref_a, ref_b, ref_c = _run_rms(a), _run_rms(b), _run_ln(c)
    torch.cuda.synchronize()
    s1 = torch.cuda.Stream(device=DEV)
    s2 = torch.cuda.Stream(device=DEV)
    s1.wait_stream(torch.cuda.current_stream(DEV))
    s2.wait_stream(torch.cuda.current_stream(DEV))
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = _run_rms(a)
        with torch.cuda.stream(s2):
            ob = _run_rms(b)
            oc = _run_ln(c)
        outs.append((oa, ob, oc))
    torch.cuda.synchronize()
    for oa, ob, oc in outs:
        for got, want in zip(oa + ob + oc, ref_a + ref_b + ref_c):
            assert torch.equal(_bits(got), _bits(want))
