"""Float64 CPU oracle for jagged HSTU attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never calls it.
"""

from .hstu_oracle import (  # noqa: F401
    attn_bwd,
    attn_bwd_kv_rows,
    attn_bwd_q_rows,
    attn_fwd,
    attn_fwd_cached,
    attn_fwd_rows,
    attn_fwd_targets,
    bucket_edges,
    bucketize,
    causal_pairs,
    chunk_bounds,
    cp_attn_blocks,
    cp_attn_bwd,
    cp_attn_fwd,
    cp_local_offsets,
    cp_rank_pairs,
    rank_chunks,
    rank_rows,
    reorder,
    reorder_index,
    silu,
    sl_keeps_whole,
    sl_select,
    sl_target_length,
    gather_rows,
    hstu_norm_gate,
    hstu_projection,
    silu_grad,
    target_mask,
    target_rows,
)
