"""Deterministic dw does not depend on how many compute units run it.

The row partition of the deterministic backward is a function of the shape
only (the route sizes it for a fixed 256 CUs, never for the device), so a
device, or a partition of one, with fewer compute units must return the same
dw bits. Each case runs in a child process whose queues are restricted to a
subset of the GPU's CUs with HSA_CU_MASK (ROCr's per-process CU mask); the
children report the bit hashes of dx and dw and the backward row kernel's
event-timed duration. The durations show that the masks took effect; the
hashes must agree across all of them.
"""
from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = [
    # (T, heads, H, w dtype, residual)
    (4096, 1, 4096, "bf16", False),      # FP32 partial rows
    (9000, 1, 2048, "f32", False),       # FP64 partial rows
    (3001, 4, 256, "f32", False),        # per-head rows, many small blocks
    (2000, 1, 6144, "bf16", True),       # residual form with dres
]
MASKS = [None, "0:0-127", "0:0-15"]


def _child() -> None:
    import numpy as np
    import torch

    import bwd_rmsnorm_fwd_02_amd as rn
    from tests import synth

    def d(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    out = {}
    for (T, heads, H, wdt, res) in CASES:
        wl = synth.make(T=T, H=H, w_dtype=wdt, seed=T + H, heads=heads, residual=res)
        w = d(wl.w.bits) if wdt == "bf16" else torch.from_numpy(wl.w.f32.copy()).cuda()
        x, dy = d(wl.x), d(wl.dy)

        def run():
            if res:
                h, _, rs = rn.rmsnorm_residual_fwd(x, d(wl.r), w, wl.eps)
                return rn.rmsnorm_residual_bwd(dy, h, rs, w, dres=d(wl.dres), deterministic=True)
            xv, dyv = x.view(T, heads, H), dy.view(T, heads, H)
            _, rs = rn.rmsnorm_fwd_strided(xv, w, wl.eps)
            return rn.rmsnorm_bwd_strided(dyv, xv, rs, w, deterministic=True)

        for _ in range(5):
            run()
        torch.cuda.synchronize()
        rn.rmsnorm_timing_read()
        rn.rmsnorm_timing_enable(True)
        dx, dw = run()
        torch.cuda.synchronize()
        timers = rn.rmsnorm_timing_read()
        rn.rmsnorm_timing_enable(False)
        n, ms = timers[1]
        out[f"{T}x{heads}x{H}"] = {
            "dw": hashlib.sha1(dw.cpu().numpy().tobytes()).hexdigest(),
            "dx": hashlib.sha1(dx.contiguous().view(torch.int16).cpu().numpy().tobytes()).hexdigest(),
            "bwd_row_us": ms / n * 1e3 if n else None,
        }
    print("RESULT " + json.dumps(out), flush=True)


def test_deterministic_dw_is_the_same_on_fewer_compute_units():
    results = {}
    for mask in MASKS:
        env = dict(os.environ)
        env.pop("HSA_CU_MASK", None)
        if mask:
            env["HSA_CU_MASK"] = mask
        print(f"child with HSA_CU_MASK={mask}", flush=True)
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "child"], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
        line = [l for l in r.stdout.splitlines() if l.startswith("RESULT ")][-1]
        results[mask] = json.loads(line[len("RESULT "):])
    full = results[None]
    for mask in MASKS[1:]:
        for case, got in results[mask].items():
            print(f"{case} mask {mask}: backward row kernel {got['bwd_row_us']:.1f} us "
                  f"(all CUs {full[case]['bwd_row_us']:.1f} us)", flush=True)
            assert got["dw"] == full[case]["dw"], f"{case}: dw differs with HSA_CU_MASK={mask}"
            assert got["dx"] == full[case]["dx"], f"{case}: dx differs with HSA_CU_MASK={mask}"
    # the masks took effect: the large cases slow down on 16 CUs
    for case in ("4096x1x4096", "9000x1x2048"):
        assert results["0:0-15"][case]["bwd_row_us"] > 3.0 * full[case]["bwd_row_us"], case


if __name__ == "__main__" and len(sys.argv) > 1 and sys.argv[1] == "child":
    sys.path.insert(0, ROOT)
    _child()
