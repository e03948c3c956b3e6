"""ctypes binding of ``libbwd_rmsnorm.so`` (the C ABI in include/rmsnorm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. torch supplies device memory and the stream.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbwd_rmsnorm.so")
# Written by the build: the code hash of the sources the library was built from.
HASH_PATH = os.path.join(HERE, "libbwd_rmsnorm.hash")

RMSN_BF16 = 0
RMSN_F32 = 1

RMSN_KIND_FWD_ROW = 1
RMSN_KIND_BWD_ROW_DET = 2
RMSN_KIND_BWD_ROW_ATOMIC = 3
RMSN_KIND_BWD_COLTASK = 4

RMSN_TIMER_FWD = 0
RMSN_TIMER_BWD_ROW = 1
RMSN_TIMER_DW_REDUCE = 2
RMSN_TIMER_BWD_SMALL = 3
RMSN_TIMER_INIT = 4
RMSN_TIMER_COUNT = 8

STATUS = {
    0: "RMSN_OK", -1: "RMSN_ERR_NULL", -2: "RMSN_ERR_DTYPE", -3: "RMSN_ERR_SHAPE",
    -4: "RMSN_ERR_ALIGN", -5: "RMSN_ERR_WORKSPACE", -6: "RMSN_ERR_OVERFLOW",
    -7: "RMSN_ERR_ALIAS", -8: "RMSN_ERR_LAUNCH", -9: "RMSN_ERR_EPS", -10: "RMSN_ERR_SCRATCH",
}

# Every symbol include/rmsnorm.h declares.
EXPORTS = [
    "rmsnorm_fwd", "rmsnorm_fwd_strided", "rmsnorm_residual_fwd", "rmsnorm_residual_fwd_strided",
    "rmsnorm_bwd_workspace_bytes", "rmsnorm_workspace_init", "rmsnorm_bwd",
    "rmsnorm_bwd_strided", "rmsnorm_bwd_recompute", "rmsnorm_residual_bwd",
    "rmsnorm_residual_bwd_strided", "rmsnorm_bwd_strided_noalloc",
    "rmsnorm_status_string",
    "rmsnorm_route_query", "rmsnorm_route_override", "rmsnorm_timing_enable",
    "rmsnorm_timing_read", "layernorm_fwd", "layernorm_bwd_workspace_bytes", "layernorm_bwd",
    "rmsnorm_bwd_partials_bytes", "rmsnorm_bwd_strided_partials",
    "rmsnorm_residual_bwd_strided_partials", "rmsnorm_dw_reduce_batch",
]


class View(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("heads", ctypes.c_int64), ("H", ctypes.c_int64),
                ("stride_t", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class DwJob(ctypes.Structure):
    _fields_ = [("partials", ctypes.c_void_p), ("partials_bytes", ctypes.c_size_t),
                ("rows", ctypes.c_int64), ("H", ctypes.c_int64), ("w_dtype", ctypes.c_int),
                ("dw", ctypes.c_void_p)]


class RouteInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("vec_per_lane", ctypes.c_int),
                ("lanes_per_row", ctypes.c_int), ("rows_per_block", ctypes.c_int),
                ("unroll", ctypes.c_int), ("block_threads", ctypes.c_int),
                ("partial_f64", ctypes.c_int), ("reduce_threads", ctypes.c_int),
                ("grid", ctypes.c_int64), ("partials", ctypes.c_int64),
                ("reduce_grid", ctypes.c_int64), ("stream_loads", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class RouteKnobs(ctypes.Structure):
    _fields_ = [("vec_per_lane", ctypes.c_int), ("unroll", ctypes.c_int),
                ("rows_per_block", ctypes.c_int), ("blocks_per_cu", ctypes.c_int),
                ("partial_f64", ctypes.c_int), ("kind", ctypes.c_int),
                ("stream_loads", ctypes.c_int)]


class RMSNormError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m bwd_rmsnorm_fwd_02_amd.build` "
            "(there is no fallback path)")
    if os.path.exists(HASH_PATH):
        # A library built from other sources may disagree with the structs
        # below (a larger route record written past a smaller one corrupts
        # the interpreter's memory), so refuse it.
        from . import build
        with open(HASH_PATH) as fh:
            built = fh.read().strip()
        if built != build.source_hash():
            raise RuntimeError(
                f"{LIB_PATH} was built from other sources (code hash {built}, sources "
                f"{build.source_hash()}): rebuild it with `python -m bwd_rmsnorm_fwd_02_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    sig = {
        "rmsnorm_fwd": [p, p, i32, f32, p, p, i64, i64, p],
        "rmsnorm_fwd_strided": [p, View, p, i32, f32, p, View, p, p],
        "rmsnorm_residual_fwd": [p, p, p, i32, f32, p, p, p, i64, i64, p],
        "rmsnorm_residual_fwd_strided": [p, View, p, View, p, i32, f32, p, View, p, View, p, p],
        "rmsnorm_bwd_workspace_bytes": [i64, i64, i32, i32],
        "rmsnorm_workspace_init": [p, sz, p],
        "rmsnorm_bwd": [p, p, p, p, i32, i32, p, p, i64, i64, p, sz, p],
        "rmsnorm_bwd_strided": [p, View, p, View, p, p, i32, i32, p, View, p, p, sz, p],
        "rmsnorm_bwd_strided_noalloc": [p, View, p, View, p, p, i32, i32, p, View, p, p],
        "rmsnorm_bwd_recompute": [p, View, p, View, p, i32, f32, i32, p, View, p, p, sz, p],
        "rmsnorm_residual_bwd": [p, p, p, p, p, i32, i32, p, p, i64, i64, p, sz, p],
        "rmsnorm_residual_bwd_strided": [p, View, p, View, p, View, p, p, i32, i32, p, View, p, p,
                                         sz, p],
        "rmsnorm_status_string": [i32],
        "rmsnorm_route_query": [i32, i64, i64, i32, i32, i32, ctypes.POINTER(RouteInfo)],
        "rmsnorm_route_override": [i32, ctypes.POINTER(RouteKnobs)],
        "rmsnorm_timing_enable": [i32],
        "rmsnorm_timing_read": [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double), i32],
        "layernorm_fwd": [p, p, p, i32, f32, p, p, p, i64, i64, p],
        "layernorm_bwd_workspace_bytes": [i64, i64, i32, i32],
        "layernorm_bwd": [p, p, p, p, p, i32, i32, p, p, p, i64, i64, p, sz, p],
        "rmsnorm_bwd_partials_bytes": [i64, i64, i32],
        "rmsnorm_bwd_strided_partials": [p, View, p, View, p, p, i32, p, View, p, sz, p],
        "rmsnorm_residual_bwd_strided_partials": [p, View, p, View, p, View, p, p, i32, p, View,
                                                  p, sz, p],
        "rmsnorm_dw_reduce_batch": [ctypes.POINTER(DwJob), i32, p],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.rmsnorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.layernorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.rmsnorm_bwd_partials_bytes.restype = ctypes.c_size_t
    lib.rmsnorm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().rmsnorm_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != 0:
        raise RMSNormError(status, status_string(status))
