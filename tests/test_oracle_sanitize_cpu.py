"""The FP64 oracle under the host sanitizers: tests/oracle_sanitize_driver.c
is built with the oracle by gcc with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts the run) and calls every oracle
entry point on shapes from empty to ragged, with each buffer allocated at its
exact size."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "rmsnorm_oracle.c"), "-I", os.path.join(ROOT, "oracle"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all shapes ok" in r.stdout
