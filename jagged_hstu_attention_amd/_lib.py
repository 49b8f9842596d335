"""ctypes loader for libhstu.so (the C ABI in include/hstu.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhstu.so")

HSTU_BF16 = 0
HSTU_FP32 = 1
HSTU_FLAG_RECOMPUTE_BWD = 1
HSTU_FLAG_SHARED_SCHEDULE = 2

STATUS = {0: "HSTU_OK", 1: "HSTU_EINVAL", 2: "HSTU_EUNSUPPORTED", 3: "HSTU_EWORKSPACE", 4: "HSTU_EHIP"}


class Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("num_seqs", ctypes.c_int64),
        ("num_heads", ctypes.c_int64),
        ("d_qk", ctypes.c_int64),
        ("d_v", ctypes.c_int64),
        ("num_buckets", ctypes.c_int64),
        ("max_seq_len", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("total_q", ctypes.c_int64),
        ("cp_size", ctypes.c_int64),
        ("cp_rank", ctypes.c_int64),
        ("sum_sq_len", ctypes.c_int64),
    ]


EXPORTS = [
    "hstu_workspace_size",
    "hstu_jagged_attn_fwd",
    "hstu_jagged_attn_fwd_targets",
    "hstu_jagged_attn_bwd",
    "hstu_cp_reorder",
    "hstu_bucket_edges",
    "hstu_last_error",
    "hstu_version",
    "hstu_timing_enable",
    "hstu_timing_reset",
    "hstu_timing_read",
    "hstu_jagged_attn_fwd_noalloc",
    "hstu_noalloc_scratch_bytes",
    "hstu_sl_select",
    "hstu_gather_rows",
    "hstu_layer_projection",
    "hstu_layer_norm_gate",
]

KERNELS = {"sched": 0, "fwd": 1, "bwd_kv": 2, "bwd_q": 3, "reorder": 4, "reduce": 5, "sl": 6, "gather": 7, "proj": 8, "norm_gate": 9}

_lib = None


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libhstu.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m jagged_hstu_attention_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, P = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(Problem)
    lib.hstu_workspace_size.argtypes = [P, ctypes.c_int]
    lib.hstu_workspace_size.restype = ctypes.c_size_t
    lib.hstu_jagged_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.hstu_jagged_attn_fwd.restype = ctypes.c_int
    lib.hstu_jagged_attn_fwd_targets.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp,
                                                 ctypes.c_size_t, vp]
    lib.hstu_jagged_attn_fwd_targets.restype = ctypes.c_int
    lib.hstu_jagged_attn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hstu_jagged_attn_fwd_noalloc.restype = ctypes.c_int
    lib.hstu_noalloc_scratch_bytes.argtypes = []
    lib.hstu_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.hstu_jagged_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.hstu_jagged_attn_bwd.restype = ctypes.c_int
    lib.hstu_cp_reorder.argtypes = [vp, vp, i64, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp]
    lib.hstu_cp_reorder.restype = ctypes.c_int
    lib.hstu_sl_select.argtypes = [vp, i64, i64, i64, ctypes.c_double, vp, vp, vp, vp, vp]
    lib.hstu_sl_select.restype = ctypes.c_int
    lib.hstu_gather_rows.argtypes = [vp, vp, i64, vp, vp, i64, vp]
    lib.hstu_gather_rows.restype = ctypes.c_int
    lib.hstu_layer_projection.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.hstu_layer_projection.restype = ctypes.c_int
    lib.hstu_layer_norm_gate.argtypes = [vp, vp, vp, i64, i64, ctypes.c_double, vp]
    lib.hstu_layer_norm_gate.restype = ctypes.c_int
    lib.hstu_bucket_edges.argtypes = [i64, ctypes.POINTER(ctypes.c_uint32)]
    lib.hstu_bucket_edges.restype = ctypes.c_int
    lib.hstu_last_error.argtypes = []
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_version.argtypes = []
    lib.hstu_version.restype = ctypes.c_int
    lib.hstu_timing_enable.argtypes = [ctypes.c_int]
    lib.hstu_timing_enable.restype = ctypes.c_int
    lib.hstu_timing_reset.argtypes = []
    lib.hstu_timing_reset.restype = ctypes.c_int
    lib.hstu_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.hstu_timing_read.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        msg = load().hstu_last_error()
        raise HstuError(status, msg.decode() if msg else "")
