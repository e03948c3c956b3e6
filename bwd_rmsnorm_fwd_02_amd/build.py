"""Build the gfx950 HIP library ``libbwd_rmsnorm.so`` in-tree with hipcc.

Every call recompiles all sources (one hipcc process per source, in
parallel) and links the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbwd_rmsnorm.so")
SOURCES = ["fwd_bf16w.hip", "fwd_f32w.hip", "bwd_bf16w.hip", "bwd_f32w.hip", "bwd_bf16w_ca.hip",
           "bwd_f32w_ca.hip", "ln_bf16w.hip",
           "ln_f32w.hip", "reduce.hip", "route.cpp", "api.cpp", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 vector instructions are disabled for every HIP source (the
# compiler would otherwise form them from plain float code).
COMMON = [
    "-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]


def _code_only(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that the hash follows the code and not its comments."""
    out = []
    i, n, quote = 0, len(src), None
    while i < n:
        c = src[i]
        if quote:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(src[i + 1])
                i += 2
                continue
            if c == quote:
                quote = None
            i += 1
        elif c in "\"'":
            quote = c
            out.append(c)
            i += 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash() -> str:
    """Hash of the code (comments and layout ignored) of every source and
    header that goes into the library. Measurement records (the HBM traffic
    files under profiles/) carry it, and are used only while it matches."""
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC))
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    with open(os.path.join(os.path.dirname(HERE), "include", "rmsnorm.h"), encoding="utf-8") as fh:
        h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(os.path.join(HERE, "libbwd_rmsnorm.hash"), "w") as fh:
        fh.write(source_hash() + "\n")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
