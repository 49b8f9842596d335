"""Jagged HSTU attention for MI355X (gfx950): thin Python binding of libhstu.so.

Every function here only marshals arguments (device pointers taken from torch
tensors, torch's current HIP stream) and calls the C ABI declared in
include/hstu.h; all computation runs in the library's HIP kernels.  torch is
used for device memory and streams only.

    out = jagged_attn_fwd(q, k, v, offsets, ts, ts_weights, max_seq_len)
    dq, dk, dv, dw = jagged_attn_bwd(dout, q, k, v, offsets, ts, ts_weights, max_seq_len)
    y, seg_offsets = cp_reorder(x, offsets, max_seq_len, cp_size)

Shapes: q, k, v, out, dout are [rows, H, d] (bf16 or fp32, contiguous, on the
GPU); offsets int64 [B+1]; ts int64 [T]; ts_weights [H, NB] in the dtype of q.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

from . import _lib
from ._lib import HSTU_BF16, HSTU_FLAG_RECOMPUTE_BWD, HSTU_FLAG_SHARED_SCHEDULE, HSTU_FP32, HstuError, Problem  # noqa: F401

__all__ = [
    "Problem", "HstuError", "HSTU_FLAG_RECOMPUTE_BWD", "HSTU_FLAG_SHARED_SCHEDULE", "problem", "workspace_size", "jagged_attn_fwd",
    "jagged_attn_fwd_targets", "jagged_attn_fwd_noalloc", "jagged_attn_bwd",
    "cp_reorder", "sl_select", "gather_rows", "layer_projection", "layer_norm_gate", "bucket_edges", "version", "library_path", "timing_enable", "timing_reset", "timing_read",
]


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> int:
    return _lib.load().hstu_version()


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HSTU_BF16
    if t.dtype == torch.float32:
        return HSTU_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def problem(q, k, v, offsets, ts_weights, max_seq_len: int, *, cp_size: int = 1, cp_rank: int = 0,
            recompute_bwd: bool = False, shared_schedule: bool = False, sum_sq_len: int = 0) -> Problem:
    """Fill the hstu_problem_t for these tensors (host metadata only).
    recompute_bwd: the memory-efficient backward (no stored score gradient).
    shared_schedule: the forward and backward of one step share one workspace
    and one schedule (see HSTU_FLAG_SHARED_SCHEDULE).  sum_sq_len: host copy of
    the sum of squared sequence lengths (0: not stated)."""
    p = Problem()
    p.dtype = _dtype_code(q)
    p.flags = (HSTU_FLAG_RECOMPUTE_BWD if recompute_bwd else 0) | (HSTU_FLAG_SHARED_SCHEDULE if shared_schedule else 0)
    p.sum_sq_len = int(sum_sq_len)
    p.num_seqs = int(offsets.shape[0]) - 1
    p.num_heads = int(q.shape[1])
    p.d_qk = int(q.shape[2])
    p.d_v = int(v.shape[2])
    p.num_buckets = int(ts_weights.shape[1])
    p.max_seq_len = int(max_seq_len)
    p.total_kv = int(k.shape[0])
    p.total_q = int(q.shape[0])
    p.cp_size = int(cp_size)
    p.cp_rank = int(cp_rank)
    return p


def workspace_size(p: Problem, backward: bool) -> int:
    n = _lib.load().hstu_workspace_size(ctypes.byref(p), 1 if backward else 0)
    if n == 0:
        _lib.check(1)
    return int(n)


def _workspace(p: Problem, backward: bool, device, workspace=None):
    torch = _torch()
    need = workspace_size(p, backward)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, int(workspace.numel() * workspace.element_size())


def jagged_attn_fwd(q, k, v, offsets, ts, ts_weights, max_seq_len: int, *, cp_size: int = 1, cp_rank: int = 0,
                    out=None, workspace=None, shared_schedule: bool = False, sum_sq_len: int = 0,
                    recompute_bwd: bool = False):
    """Forward of jagged HSTU attention; returns out [total_q, H, d_v].
    shared_schedule: also build the backward's work lists in `workspace` (sized
    for the backward) for a jagged_attn_bwd(..., shared_schedule=True) with the
    same workspace to reuse; the two calls describe the same problem, so
    recompute_bwd states which backward follows."""
    torch = _torch()
    p = problem(q, k, v, offsets, ts_weights, max_seq_len, cp_size=cp_size, cp_rank=cp_rank,
                shared_schedule=shared_schedule, sum_sq_len=sum_sq_len, recompute_bwd=recompute_bwd)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    ws, ws_bytes = _workspace(p, False, q.device, workspace)
    lib = _lib.load()
    _lib.check(lib.hstu_jagged_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets), _ptr(ts),
                                        _ptr(ts_weights), _ptr(out), _ptr(ws), ws_bytes, _stream(q.device)))
    return out


def jagged_attn_fwd_noalloc(q, k, v, offsets, ts, ts_weights, max_seq_len: int, *, cp_size: int = 1,
                            cp_rank: int = 0, out=None):
    """Forward through the entry point that allocates nothing: its scratch is
    the library's static per-GPU array (calls on one GPU must not overlap).
    Returns out [total_q, H, d_v] (allocated here by torch unless given)."""
    torch = _torch()
    p = problem(q, k, v, offsets, ts_weights, max_seq_len, cp_size=cp_size, cp_rank=cp_rank)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    lib = _lib.load()
    _lib.check(lib.hstu_jagged_attn_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                                _ptr(ts), _ptr(ts_weights), _ptr(out), _stream(q.device)))
    return out


def jagged_attn_fwd_targets(q, k, v, offsets, num_targets, ts, ts_weights, max_seq_len: int, *,
                            q_targets_only: bool = False, out=None, workspace=None):
    """Forward with candidates: the last num_targets[b] rows of sequence b
    attend to its history rows and to themselves only.  q_targets_only: q
    holds just those candidate rows (k, v, ts cover all rows).  Returns out
    [q.shape[0], H, d_v]."""
    torch = _torch()
    p = problem(q, k, v, offsets, ts_weights, max_seq_len)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=q.dtype, device=q.device)
    ws, ws_bytes = _workspace(p, False, q.device, workspace)
    lib = _lib.load()
    _lib.check(lib.hstu_jagged_attn_fwd_targets(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                                _ptr(num_targets), 1 if q_targets_only else 0, _ptr(ts),
                                                _ptr(ts_weights), _ptr(out), _ptr(ws), ws_bytes,
                                                _stream(q.device)))
    return out


def jagged_attn_bwd(dout, q, k, v, offsets, ts, ts_weights, max_seq_len: int, *, cp_size: int = 1,
                    cp_rank: int = 0, dq=None, dk=None, dv=None, dw=None, workspace=None,
                    recompute: bool = False, shared_schedule: bool = False, sum_sq_len: int = 0):
    """Backward; returns (dq, dk, dv, d_ts_weights) with d_ts_weights in fp32.
    recompute: memory-efficient form (the dQ pass recomputes the score
    gradient instead of reading it from the workspace).  shared_schedule: reuse
    the work lists the preceding forward built in the same workspace."""
    torch = _torch()
    p = problem(q, k, v, offsets, ts_weights, max_seq_len, cp_size=cp_size, cp_rank=cp_rank,
                recompute_bwd=recompute, shared_schedule=shared_schedule, sum_sq_len=sum_sq_len)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dw = torch.empty(ts_weights.shape, dtype=torch.float32, device=q.device) if dw is None else dw
    ws, ws_bytes = _workspace(p, True, q.device, workspace)
    lib = _lib.load()
    _lib.check(lib.hstu_jagged_attn_bwd(ctypes.byref(p), _ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(offsets),
                                        _ptr(ts), _ptr(ts_weights), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw),
                                        _ptr(ws), ws_bytes, _stream(q.device)))
    return dq, dk, dv, dw


def cp_reorder(x, offsets, max_seq_len: int, cp_size: int, *, inverse: bool = False, out=None,
               out_offsets=None, want_offsets: bool = True) -> Tuple[object, Optional[object]]:
    """Load-balanced chunk-pair row permutation of x [rows, ...] (bit-exact).

    Returns (y, seg_offsets) where seg_offsets (int64 [cp_size*B + 1], or None)
    delimits the rank-major segments (rank r, sequence b) -> index r*B + b."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    B = int(offsets.shape[0]) - 1
    if want_offsets and out_offsets is None:
        out_offsets = torch.empty(cp_size * B + 1, dtype=torch.int64, device=x.device)
    row_bytes = x.element_size() * math.prod(x.shape[1:])
    lib = _lib.load()
    _lib.check(lib.hstu_cp_reorder(_ptr(x), _ptr(out), row_bytes, _ptr(offsets), B, int(x.shape[0]),
                                   int(max_seq_len), int(cp_size), 1 if inverse else 0,
                                   _ptr(out_offsets) if out_offsets is not None else None, _stream(x.device)))
    return out, out_offsets


def sl_select(offsets, max_seq_len: int, alpha: float, seq_uniform, token_keys=None, *, out_offsets=None,
              out_index=None):
    """Stochastic Length selection.  offsets int64 [B+1]; seq_uniform float32
    [B] (keep-whole draws in [0, 1)); token_keys uint32-valued int32 [T] (the
    L smallest are kept) or None (recency).  Returns (out_offsets [B+1],
    out_index [T]); only the first out_offsets[B] entries of out_index are
    written (the count stays on the device)."""
    torch = _torch()
    B = int(offsets.shape[0]) - 1
    T = int(token_keys.shape[0]) if token_keys is not None else None
    if out_offsets is None:
        out_offsets = torch.empty(B + 1, dtype=torch.int64, device=offsets.device)
    if out_index is None:
        if T is None:
            raise ValueError("out_index must be given (or token_keys, whose length is the row count)")
        out_index = torch.empty(T, dtype=torch.int64, device=offsets.device)
    total = int(out_index.shape[0])
    _lib.check(_lib.load().hstu_sl_select(_ptr(offsets), B, total, int(max_seq_len), float(alpha), _ptr(seq_uniform),
                                          _ptr(token_keys), _ptr(out_offsets), _ptr(out_index),
                                          _stream(offsets.device)))
    return out_offsets, out_index


def gather_rows(x, index, count, *, out=None):
    """out[i] = x[index[i]] for i < count[0] (count: a one-element device
    tensor, e.g. out_offsets[-1:]); rows past the count are left as they are.
    out defaults to a tensor of x's shape."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(x)
    row_bytes = x.element_size() * math.prod(x.shape[1:])
    _lib.check(_lib.load().hstu_gather_rows(_ptr(x), _ptr(out), row_bytes, _ptr(index), _ptr(count),
                                            min(int(index.shape[0]), int(out.shape[0])), _stream(x.device)))
    return out


def layer_projection(x, w, num_heads: int, d_qk: int, d_v: int, *, out=None):
    """[U V Q K] = SiLU(x wᵀ) split per head: x [T, d_model] bf16, w [H (2 d_v +
    2 d_qk), d_model] bf16.  Returns (u, v, q, k) as [T, H, d] tensors."""
    torch = _torch()
    T = int(x.shape[0])
    if out is None:
        out = (torch.empty((T, num_heads, d_v), dtype=x.dtype, device=x.device),
               torch.empty((T, num_heads, d_v), dtype=x.dtype, device=x.device),
               torch.empty((T, num_heads, d_qk), dtype=x.dtype, device=x.device),
               torch.empty((T, num_heads, d_qk), dtype=x.dtype, device=x.device))
    u, v, q, k = out
    _lib.check(_lib.load().hstu_layer_projection(_ptr(x), _ptr(w), T, int(x.shape[1]), int(num_heads), int(d_qk),
                                                 int(d_v), _ptr(u), _ptr(v), _ptr(q), _ptr(k), _stream(x.device)))
    return u, v, q, k


def layer_norm_gate(o, u, *, eps: float = 1e-6, out=None):
    """Norm(o) ⊙ u per row: o, u [T, H, d_v] bf16 (or [T, width]); returns
    [T, H * d_v]."""
    torch = _torch()
    T = int(o.shape[0])
    width = math.prod(o.shape[1:])
    if out is None:
        out = torch.empty((T, width), dtype=o.dtype, device=o.device)
    _lib.check(_lib.load().hstu_layer_norm_gate(_ptr(o), _ptr(u), _ptr(out), T, width, float(eps), _stream(o.device)))
    return out


def bucket_edges(num_buckets: int):
    """The library's integer edge table E[0..NB] (host computation) as a list."""
    arr = (ctypes.c_uint32 * (num_buckets + 1))()
    _lib.check(_lib.load().hstu_bucket_edges(int(num_buckets), arr))
    return list(arr)


def timing_enable(on: bool = True) -> None:
    """Record HIP events around every kernel launch (per-kernel timing)."""
    _lib.check(_lib.load().hstu_timing_enable(1 if on else 0))


def timing_reset() -> None:
    _lib.check(_lib.load().hstu_timing_reset())


def timing_read(kernel: str):
    """(total milliseconds, launches) accumulated for one kernel since the last
    reset; kernel is one of sched, fwd, bwd_kv, bwd_q, reorder."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _lib.check(_lib.load().hstu_timing_read(_lib.KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
