"""ctypes loader for libmoe_vs.so (the C ABI declared in include/moe_vs.h).

Only argument marshalling lives here: every step of the grouped GEMM runs in
the HIP library.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_vs.so")

MOE_OK = 0
MOE_F32 = 0
MOE_BF16 = 1
MOE_LAYOUT_CONTIGUOUS = 0
MOE_LAYOUT_MASKED = 1
MOE_NUM_BM = 4
BM_VALUES = (32, 64, 128, 256)
MOE_COMBINE_AUTO = 0
MOE_COMBINE_ATOMIC = 1
MOE_COMBINE_RANKED = 2


class MoeSchedule(ctypes.Structure):
    """Mirror of ``struct moe_schedule``."""

    _fields_ = [
        ("T", ctypes.c_int64),
        ("S", ctypes.c_int64),
        ("R", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("block_start", ctypes.c_void_p),
        ("expert_order", ctypes.c_void_p),
        ("row_to_assign", ctypes.c_void_p),
        ("row_to_token", ctypes.c_void_p),
        ("row_weight", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
        ("phases", ctypes.c_int32),
        ("phase_counts", ctypes.c_void_p),
        ("phase_offsets", ctypes.c_void_p),
        ("phase_block_start", ctypes.c_void_p),
        ("phase_row_to_assign", ctypes.c_void_p),
        ("phase_row_to_token", ctypes.c_void_p),
        ("phase_row_weight", ctypes.c_void_p),
        ("phase_sync", ctypes.c_void_p),
        ("weighted", ctypes.c_int32),
        ("dw_queue", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SCHED_P = ctypes.POINTER(MoeSchedule)

SIGNATURES = {
    "moe_schedule_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32]),
    "moe_build_schedule": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _SCHED_P, _P]),
    "moe_build_schedule_noalloc": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _SCHED_P, _P]),
    "grouped_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P]),
    "moe_fused_fwd": (ctypes.c_int, [_P, _P, _SCHED_P, _P, _I64, _I64, _I32, _P]),
    "moe_fused_fwd_fp8": (ctypes.c_int, [_P, _P, _P, _P, _SCHED_P, _P, _I64, _I64, _P]),
    "moe_fused_fwd_mx": (ctypes.c_int, [_P, _P, _P, _P, _SCHED_P, _P, _I64, _I64, _P]),
    "moe_gated_ffn_fwd": (ctypes.c_int, [_P, _P, _P, _SCHED_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "moe_gated_ffn_bwd_workspace_bytes": (_SZ, [_SCHED_P, _I64]),
    "moe_gated_ffn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _SCHED_P, _P, _P, _P, _P, _P, _P, _I64,
                                         _I64, _I64, _I32, _P, _SZ, _P]),
    "moe_fused_bwd_workspace_bytes": (_SZ, [_SCHED_P, _I64, _I64, _I32]),
    "moe_fused_bwd": (ctypes.c_int, [_P, _P, _P, _SCHED_P, _P, _P, _P, _I64, _I64, _I32, _P, _SZ, _P]),
    "moe_tile_map": (ctypes.c_int, [_SCHED_P, _I64, _I32, _I32, _P, _P, _P, _I64, _P]),
    "moe_set_tile_rows": (ctypes.c_int, [_I32]),
    "moe_set_combine": (ctypes.c_int, [_I32]),
    "moe_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_version": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"HIP library not found at {path}; build it with "
                    "`python -m moe_variable_size_amd.build` (hipcc, gfx950)")
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().moe_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
