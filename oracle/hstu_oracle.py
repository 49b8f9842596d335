"""Float64 CPU oracle for jagged HSTU attention (test infrastructure only).

This module is the independent reference that the HIP path is checked against.
It is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
library (``jagged_hstu_attention_amd``) and imports nothing from it.

Sources (the pages; titles abbreviated):

* [CP]   "Scaling Generative Recommendations with Context Parallelism on
         Hierarchical Sequential Transducers" (arXiv 2508.04711, LaTeX source).
* [HSTU] "Actions Speak Louder than Words: Trillion-Parameter Sequential
         Transducers for Generative Recommendations" (arXiv 2402.17152v3 summary).
* [REV]  Pith review of the CP paper (pith.science).

What is computed, with the readings taken where the pages are open
(each reading is listed again in the design notes):

1. Attention, [CP] §2.1 HSTUAttention equation:
   O = Mask(SiLU((Q Kᵀ + Bias) / sqrt(d_k))) V.  No softmax or any other
   normalisation of the weights ([HSTU] §3.1, pointwise aggregated attention).
   d_k is the Q/K width.  The bias sits inside the division (equation as set).
   SiLU(x) = x * sigmoid(x).  Mask is causal, including the diagonal, and
   block-diagonal over the jagged sequences ([CP] §2.3 causal mask).
2. Bias, [CP] §2.1 (timestamp bias paragraph): a difference of timestamps,
   a transformation, then a grouping into bucket indices that select from the
   learnable ``ts_weights``.  Reading: the difference is taken per query/key
   pair (Δ = ts_query - ts_key; [REV] speaks of biases for query-key pairs),
   the transformation is log2|Δ|, and the grouping is NB equal-width bins of
   log2|Δ| over [0, 32), i.e. bucket(Δ) = #{k in [1, NB): |Δ| >= E_k} with
   E_k = ceil(2^(32 k / NB)).  The integer edge table is the definition; it is
   computed here exactly with Python integers.
3. Backward: plain calculus of 1-2 (gradients w.r.t. Q, K, V and ts_weights);
   the weights are never normalised, so no statistics are needed.
4. Context-parallel share, [CP] §2.3 load balancing: each sequence is cut into
   2C mini-chunks and rank r holds chunks r and 2C-1-r.  Chunk k of a length-L
   sequence is rows [floor(kL/2C), floor((k+1)L/2C)) (reading for L not divisible
   by 2C).  A rank's query rows keep their global positions and global
   timestamps, and attend to their causal key prefix of the full sequence.
5. Reorder, [CP] §2.3 (memory-reordering data shuffle): the rank-major
   permutation of rows; rank, then sequence, then chunk r then chunk 2C-1-r.
8. HSTU layer steps either side of the attention, [HSTU] §3 (residual
   layers of pointwise projection, spatial aggregation and pointwise
   transformation; the interaction Norm(A(X)V(X)) ⊙ U(X)).  Readings: the
   projection is one linear map without bias followed by SiLU, split into
   U, V, Q, K in that order: [U V Q K] = SiLU(X Wᵀ) with W [H(2 d_v +
   2 d_qk), d_model] (the layout of a linear layer's weight); Norm is layer
   normalisation over each row's H d_v attention outputs, eps = 1e-6, no
   learned scale or shift; the step returns Norm(O) ⊙ U, O the attention
   output.  The output projection and residual add are not printed and are
   not part of it.
7. Stochastic Length, [HSTU] §3.2 and §4.2 (sequence sparsity by subsequence
   selection; at alpha = 1.6 a length-4096 history becomes length 776 most of
   the time) and App. E (the subsequence is chosen by recency, at random, or
   by feature weights).  Readings: a sequence of length n is cut to
   L = floor(n^(alpha/2)) rows (4096^0.8 = 776.05; the power carries a 2^-40
   relative tolerance so that a float alpha such as 1.2 gives 32^0.6 = 8,
   not the 7 its binary value would), except that with
   probability n^(alpha-2) it is kept whole (so the printed case is cut with
   probability 1 - 4096^-0.4 = 0.964, "most of the time"); the draw is an
   input u_b in [0, 1), kept whole iff u_b < n^(alpha-2).  The kept rows are
   the last L (recency) or the L with the smallest random keys, ties broken by
   position (random, the keys are inputs), in their original order.
   Feature-weighted selection needs features the pages do not define.

All floating-point arithmetic is float64; timestamps stay exact integers.
Every function takes the exact values the device sees (bf16 inputs widened
exactly to float64).
"""

from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np

BUCKET_LOG2_SPAN = 32  # the bins of log2|Δ| cover [0, 32)


# --------------------------------------------------------------------------
# 2. Timestamp bucketing ([CP] §2.1, timestamp bias paragraph)
# --------------------------------------------------------------------------

def _ceil_root_pow2(exponent: int, n: int) -> int:
    """Smallest integer x >= 0 with x**n >= 2**exponent, exactly."""
    target = 1 << exponent
    x = int(math.ceil(2.0 ** (exponent / n)))
    while x > 0 and (x - 1) ** n >= target:
        x -= 1
    while x ** n < target:
        x += 1
    return x


def bucket_edges(num_buckets: int) -> List[int]:
    """Exact integer edges E_k = ceil(2^(32 k / NB)) for k = 1 .. NB-1.

    Edge k is the smallest integer x with x^NB >= 2^(32 k).  The returned list
    has NB-1 entries (index k-1 holds E_k); it is non-decreasing and may repeat
    values for small k when NB > 32.
    """
    if num_buckets < 1:
        raise ValueError("num_buckets must be >= 1")
    return [_ceil_root_pow2(BUCKET_LOG2_SPAN * k, num_buckets) for k in range(1, num_buckets)]


def bucketize(delta: np.ndarray, num_buckets: int) -> np.ndarray:
    """bucket(Δ) = #{k in [1, NB): |Δ| >= E_k}, exact on int64 Δ (|Δ| < 2^63)."""
    delta = np.asarray(delta, dtype=np.int64)
    mag = np.abs(delta)
    edges = np.asarray(bucket_edges(num_buckets), dtype=np.int64)
    if edges.size == 0:
        return np.zeros(mag.shape, dtype=np.int64)
    return np.searchsorted(edges, mag, side="right").astype(np.int64)


# --------------------------------------------------------------------------
# 1. Forward ([CP] §2.1 HSTUAttention equation)
# --------------------------------------------------------------------------

def silu(x):
    return x / (1.0 + np.exp(-x))


def silu_grad(x):
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 + x * (1.0 - s))


def _seq_scores(qb, kb, tsq, tsk, wh, nb, alpha):
    """s = alpha * (q·k + w[bucket(ts_q - ts_k)]) for one (sequence, head)."""
    raw = qb @ kb.T
    bucket = bucketize(tsq[:, None] - tsk[None, :], nb)
    return alpha * (raw + wh[bucket]), bucket


def attn_fwd(q, k, v, offsets, ts, w, num_buckets) -> np.ndarray:
    """Jagged HSTU attention forward.

    q, k: [T, H, d_qk]; v: [T, H, d_v]; offsets: int64 [B+1]; ts: int64 [T];
    w: [H, NB].  Returns O [T, H, d_v] in float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    ts = np.asarray(ts, np.int64)
    T, H, dqk = q.shape
    alpha = 1.0 / math.sqrt(dqk)
    out = np.zeros((T, H, v.shape[2]), dtype=np.float64)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi <= lo:
            continue
        n = hi - lo
        mask = np.tril(np.ones((n, n), dtype=bool))
        for h in range(H):
            s, _ = _seq_scores(q[lo:hi, h], k[lo:hi, h], ts[lo:hi], ts[lo:hi], w[h],
                               num_buckets, alpha)
            a = np.where(mask, silu(s), 0.0)
            out[lo:hi, h] = a @ v[lo:hi, h]
    return out


# --------------------------------------------------------------------------
# 3. Backward
# --------------------------------------------------------------------------

def attn_bwd(dout, q, k, v, offsets, ts, w, num_buckets):
    """Gradients of sum(dout * O) w.r.t. q, k, v and w (float64).

    With s = alpha*(q·k + w[bucket]) and a = SiLU(s)*mask:
      dP = dO Vᵀ;  G = alpha * dP * SiLU'(s) * mask;
      dV = aᵀ dO;  dQ = G K;  dK = Gᵀ Q;  dW[h, b] = sum of G over pairs in bucket b.
    Returns (dq, dk, dv, dw) with dw of shape [H, NB].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    dout = np.asarray(dout, np.float64)
    ts = np.asarray(ts, np.int64)
    T, H, dqk = q.shape
    alpha = 1.0 / math.sqrt(dqk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dw = np.zeros((H, num_buckets), dtype=np.float64)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi <= lo:
            continue
        n = hi - lo
        mask = np.tril(np.ones((n, n), dtype=bool))
        for h in range(H):
            s, bucket = _seq_scores(q[lo:hi, h], k[lo:hi, h], ts[lo:hi], ts[lo:hi], w[h],
                                    num_buckets, alpha)
            a = np.where(mask, silu(s), 0.0)
            dp = dout[lo:hi, h] @ v[lo:hi, h].T
            g = np.where(mask, alpha * dp * silu_grad(s), 0.0)
            dv[lo:hi, h] = a.T @ dout[lo:hi, h]
            dq[lo:hi, h] = g @ k[lo:hi, h]
            dk[lo:hi, h] = g.T @ q[lo:hi, h]
            dw[h] += np.bincount(bucket[mask], weights=g[mask], minlength=num_buckets)
    return dq, dk, dv, dw


# --------------------------------------------------------------------------
# 4. Context-parallel share ([CP] §2.3, load-balanced mini-chunks)
# --------------------------------------------------------------------------

def chunk_bounds(length: int, cp_size: int, chunk: int) -> Tuple[int, int]:
    """Rows [floor(k L / 2C), floor((k+1) L / 2C)) of mini-chunk k."""
    nchunks = 2 * cp_size
    return (chunk * length) // nchunks, ((chunk + 1) * length) // nchunks


def rank_chunks(cp_size: int, rank: int) -> Tuple[int, int]:
    """Rank r holds mini-chunks r and 2C-1-r."""
    return rank, 2 * cp_size - 1 - rank


def reorder_index(offsets: Sequence[int], cp_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row permutation of the load-balanced layout, by explicit nested loops.

    Returns (idx, out_offsets): output row i is input row idx[i]; out_offsets
    has cp_size*B + 1 entries, one segment per (rank, sequence).
    """
    B = len(offsets) - 1
    idx: List[int] = []
    out_offsets = [0]
    for r in range(cp_size):
        for b in range(B):
            start = int(offsets[b])
            length = int(offsets[b + 1]) - start
            for c in rank_chunks(cp_size, r):
                c0, c1 = chunk_bounds(length, cp_size, c)
                for row in range(c0, c1):
                    idx.append(start + row)
            out_offsets.append(len(idx))
    return np.asarray(idx, dtype=np.int64), np.asarray(out_offsets, dtype=np.int64)


def reorder(x: np.ndarray, offsets, cp_size: int, inverse: bool = False):
    """Apply the load-balanced permutation to the leading (row) axis of x."""
    idx, out_offsets = reorder_index(offsets, cp_size)
    x = np.asarray(x)
    if not inverse:
        return x[idx], out_offsets
    out = np.empty_like(x)
    out[idx] = x
    return out, out_offsets


def rank_rows(offsets, cp_size: int, rank: int):
    """For one rank: per sequence, the list of (global row, position) it holds,
    in the rank's local order (chunk r then chunk 2C-1-r)."""
    rows = []
    for b in range(len(offsets) - 1):
        start = int(offsets[b])
        length = int(offsets[b + 1]) - start
        seq_rows = []
        for c in rank_chunks(cp_size, rank):
            c0, c1 = chunk_bounds(length, cp_size, c)
            seq_rows.extend((start + p, p) for p in range(c0, c1))
        rows.append(seq_rows)
    return rows


def cp_local_offsets(offsets, cp_size: int, rank: int) -> np.ndarray:
    lens = [len(r) for r in rank_rows(offsets, cp_size, rank)]
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(lens)
    return out


def cp_attn_fwd(q_local, k, v, offsets, ts, w, num_buckets, cp_size, rank):
    """One rank's share of the forward.

    q_local: [Tr, H, d_qk], the rank's query rows in local order; k, v, ts are
    the full global tensors.  Each local row at global position p attends to
    keys 0..p of its sequence with global timestamps.  Returns [Tr, H, d_v].
    """
    q_local = np.asarray(q_local, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    ts = np.asarray(ts, np.int64)
    H, dqk = q_local.shape[1], q_local.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    out = np.zeros((q_local.shape[0], H, v.shape[2]), dtype=np.float64)
    local = 0
    for b, seq_rows in enumerate(rank_rows(offsets, cp_size, rank)):
        start = int(offsets[b])
        for (grow, p) in seq_rows:
            keys = slice(start, start + p + 1)
            for h in range(H):
                s, _ = _seq_scores(q_local[local:local + 1, h], k[keys, h],
                                   ts[grow:grow + 1], ts[keys], w[h], num_buckets, alpha)
                out[local, h] = silu(s)[0] @ v[keys, h]
            local += 1
    return out


def cp_attn_bwd(dout_local, q_local, k, v, offsets, ts, w, num_buckets, cp_size, rank):
    """One rank's share of the backward.

    Returns (dq_local [Tr,H,d_qk], dk [T,H,d_qk], dv [T,H,d_v], dw [H,NB]) where
    dk, dv and dw are this rank's partial sums (zeros for keys no local row
    reaches); summing them over all ranks gives the unsharded gradients.
    """
    q_local = np.asarray(q_local, np.float64)
    dout_local = np.asarray(dout_local, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    ts = np.asarray(ts, np.int64)
    H, dqk = q_local.shape[1], q_local.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    dq = np.zeros_like(q_local)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dw = np.zeros((H, num_buckets), dtype=np.float64)
    local = 0
    for b, seq_rows in enumerate(rank_rows(offsets, cp_size, rank)):
        start = int(offsets[b])
        for (grow, p) in seq_rows:
            keys = slice(start, start + p + 1)
            for h in range(H):
                s, bucket = _seq_scores(q_local[local:local + 1, h], k[keys, h],
                                        ts[grow:grow + 1], ts[keys], w[h], num_buckets, alpha)
                s = s[0]
                bucket = bucket[0]
                a = silu(s)
                dp = v[keys, h] @ dout_local[local, h]
                g = alpha * dp * silu_grad(s)
                dv[keys, h] += np.outer(a, dout_local[local, h])
                dq[local, h] = g @ k[keys, h]
                dk[keys, h] += np.outer(g, q_local[local, h])
                dw[h] += np.bincount(bucket, weights=g, minlength=num_buckets)
            local += 1
    return dq, dk, dv, dw


def cp_attn_blocks(dout_local, q_local, k, v, offsets, ts, w, num_buckets, cp_size, rank):
    """One rank's share, forward and backward, as one masked block per
    (sequence, head): the rank's query rows of a sequence (chunk r then chunk
    2C-1-r, at their global positions p) against the keys 0 .. max p of that
    sequence, key j visible to row p iff j <= p.  The same quantities as
    cp_attn_fwd and cp_attn_bwd (and the same readings), with the rows of a
    sequence stacked into one matrix instead of looped over.

    Returns (out_local, dq_local, dk, dv, dw); dk, dv, dw are the rank's
    partial sums as in cp_attn_bwd.
    """
    q_local = np.asarray(q_local, np.float64)
    dout_local = np.asarray(dout_local, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    ts = np.asarray(ts, np.int64)
    H, dqk = q_local.shape[1], q_local.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    out = np.zeros((q_local.shape[0], H, v.shape[2]), dtype=np.float64)
    dq = np.zeros_like(q_local)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dw = np.zeros((H, num_buckets), dtype=np.float64)
    local = 0
    for b, seq_rows in enumerate(rank_rows(offsets, cp_size, rank)):
        n = len(seq_rows)
        if n == 0:
            continue
        start = int(offsets[b])
        grows = np.array([g for g, _ in seq_rows], dtype=np.int64)
        pos = np.array([p for _, p in seq_rows], dtype=np.int64)
        nk = int(pos.max()) + 1
        keys = slice(start, start + nk)
        mask = np.arange(nk)[None, :] <= pos[:, None]
        rows = slice(local, local + n)
        for h in range(H):
            s, bucket = _seq_scores(q_local[rows, h], k[keys, h], ts[grows], ts[keys], w[h], num_buckets, alpha)
            a = np.where(mask, silu(s), 0.0)
            out[rows, h] = a @ v[keys, h]
            dp = dout_local[rows, h] @ v[keys, h].T
            g = np.where(mask, alpha * dp * silu_grad(s), 0.0)
            dv[keys, h] += a.T @ dout_local[rows, h]
            dq[rows, h] = g @ k[keys, h]
            dk[keys, h] += g.T @ q_local[rows, h]
            dw[h] += np.bincount(bucket[mask], weights=g[mask], minlength=num_buckets)
        local += n
    return out, dq, dk, dv, dw


# --------------------------------------------------------------------------
# 7. Stochastic Length ([HSTU] §3.2, §4.2, App. E)
# --------------------------------------------------------------------------

def _pow_exact(n: int, exponent: Fraction) -> Decimal:
    """n ** exponent to 60 significant digits (the exponent is an exact
    rational: the float the caller passed, halved or shifted exactly)."""
    with localcontext() as ctx:
        ctx.prec = 60
        return Decimal(n) ** (Decimal(exponent.numerator) / Decimal(exponent.denominator))


# alpha arrives as a binary float (1.2 is not 6/5), so n^(alpha/2) at a
# perfect power (32^0.6 = 8) can fall a hair below the integer the caller
# means; a relative tolerance of 2^-40 on the power absorbs that.
SL_REL_TOL = Fraction(1, 1 << 40)


def sl_target_length(n: int, alpha: float) -> int:
    """L = floor(n^(alpha/2) (1 + 2^-40)), at most n."""
    if n <= 0:
        return 0
    with localcontext() as ctx:
        ctx.prec = 60
        x = _pow_exact(n, Fraction(alpha) / 2) * (1 + Decimal(SL_REL_TOL.numerator) / Decimal(SL_REL_TOL.denominator))
    return min(int(math.floor(x)), n)


def sl_keeps_whole(n: int, alpha: float, u: float) -> bool:
    """The sequence is kept whole iff u < n^(alpha-2) (so with probability
    n^(alpha-2) for u ~ U[0, 1)), or when the cut would not shorten it."""
    if n <= 1 or sl_target_length(n, alpha) >= n:
        return True
    with localcontext() as ctx:
        ctx.prec = 60
        return Decimal(float(u)) < _pow_exact(n, Fraction(alpha) - 2)


def sl_select(offsets, alpha: float, seq_uniform, token_keys=None):
    """Rows kept by Stochastic Length, sequence by sequence.

    offsets int64 [B+1]; seq_uniform [B] (the keep-whole draws); token_keys
    [T] uint32 (random selection) or None (recency: the last L rows).
    Returns (out_offsets [B+1], index [T_out]): output row i is input row
    index[i]."""
    out_off = [0]
    idx = []
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        n = hi - lo
        if n <= 0:
            out_off.append(len(idx))
            continue
        if sl_keeps_whole(n, alpha, float(seq_uniform[b])):
            kept = list(range(lo, hi))
        else:
            L = sl_target_length(n, alpha)
            if token_keys is None:
                kept = list(range(hi - L, hi))
            else:
                order = sorted(range(lo, hi), key=lambda r: (int(token_keys[r]), r))
                kept = sorted(order[:L])
        idx.extend(kept)
        out_off.append(len(idx))
    return np.asarray(out_off, dtype=np.int64), np.asarray(idx, dtype=np.int64)


def gather_rows(x, index):
    """out[i] = x[index[i]] (rows of any shape and dtype, bytes unchanged)."""
    return np.asarray(x)[np.asarray(index, dtype=np.int64)]


# --------------------------------------------------------------------------
# 8. HSTU layer steps ([HSTU] §3: pointwise projection; Norm(A(X)V(X)) ⊙ U(X))
# --------------------------------------------------------------------------

LAYER_NORM_EPS = 1e-6


def hstu_projection(x, w, num_heads: int, d_qk: int, d_v: int):
    """[U V Q K] = SiLU(x wᵀ): x [T, d_model], w [H (2 d_v + 2 d_qk), d_model].
    Returns U, V [T, H, d_v] and Q, K [T, H, d_qk] (float64)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    h = silu(x @ w.T)
    T = x.shape[0]
    cu, cv, cq = num_heads * d_v, 2 * num_heads * d_v, 2 * num_heads * d_v + num_heads * d_qk
    u = h[:, :cu].reshape(T, num_heads, d_v)
    v = h[:, cu:cv].reshape(T, num_heads, d_v)
    q = h[:, cv:cq].reshape(T, num_heads, d_qk)
    k = h[:, cq:].reshape(T, num_heads, d_qk)
    return u, v, q, k


def hstu_norm_gate(o, u, eps: float = LAYER_NORM_EPS):
    """Norm(O) ⊙ U: o, u [T, H, d_v]; layer norm over each row's H d_v
    values (mean 0, variance 1, biased variance, eps inside the root).
    Returns [T, H d_v] (float64)."""
    o = np.asarray(o, np.float64)
    u = np.asarray(u, np.float64)
    T = o.shape[0]
    flat = o.reshape(T, -1)
    mean = flat.mean(axis=1, keepdims=True)
    var = ((flat - mean) ** 2).mean(axis=1, keepdims=True)
    return (flat - mean) / np.sqrt(var + eps) * u.reshape(T, -1)


# --------------------------------------------------------------------------
# Counting (for the measurement: causal-effective pairs)
# --------------------------------------------------------------------------

def causal_pairs(lengths) -> int:
    """Number of (i, j) with j <= i inside each sequence, summed."""
    return int(sum(int(n) * (int(n) + 1) // 2 for n in lengths))


def cp_rank_pairs(lengths, cp_size: int, rank: int) -> int:
    """Causal pairs whose query row belongs to the rank's two mini-chunks."""
    total = 0
    for n in lengths:
        for c in rank_chunks(cp_size, rank):
            c0, c1 = chunk_bounds(int(n), cp_size, c)
            total += sum(p + 1 for p in range(c0, c1))
    return total


# --------------------------------------------------------------------------
# Per-row forms, for checking sampled outputs of large problems.  Same
# arithmetic as above, restricted to the requested rows.
# --------------------------------------------------------------------------

def _row_seq(offsets, row):
    b = int(np.searchsorted(np.asarray(offsets), row, side="right")) - 1
    return b, int(offsets[b]), int(offsets[b + 1])


def attn_fwd_rows(q, k, v, offsets, ts, w, num_buckets, rows):
    """O[rows] of attn_fwd (all heads): [len(rows), H, d_v]."""
    q = np.asarray(q)
    H, dqk = q.shape[1], q.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    out = np.zeros((len(rows), H, v.shape[2]), dtype=np.float64)
    for n, i in enumerate(rows):
        _, lo, _ = _row_seq(offsets, i)
        keys = slice(lo, i + 1)
        for h in range(H):
            s, _ = _seq_scores(np.asarray(q[i:i + 1, h], np.float64), np.asarray(k[keys, h], np.float64),
                               ts[i:i + 1], ts[keys], np.asarray(w[h], np.float64), num_buckets, alpha)
            out[n, h] = silu(s)[0] @ np.asarray(v[keys, h], np.float64)
    return out


def attn_bwd_q_rows(dout, q, k, v, offsets, ts, w, num_buckets, rows):
    """dQ[rows] of attn_bwd: [len(rows), H, d_qk]."""
    H, dqk = q.shape[1], q.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    dq = np.zeros((len(rows), H, dqk), dtype=np.float64)
    for n, i in enumerate(rows):
        _, lo, _ = _row_seq(offsets, i)
        keys = slice(lo, i + 1)
        for h in range(H):
            kk = np.asarray(k[keys, h], np.float64)
            s, _ = _seq_scores(np.asarray(q[i:i + 1, h], np.float64), kk, ts[i:i + 1], ts[keys],
                               np.asarray(w[h], np.float64), num_buckets, alpha)
            dp = np.asarray(v[keys, h], np.float64) @ np.asarray(dout[i, h], np.float64)
            g = alpha * dp * silu_grad(s[0])
            dq[n, h] = g @ kk
    return dq


def attn_bwd_kv_rows(dout, q, k, v, offsets, ts, w, num_buckets, rows):
    """(dK[rows], dV[rows]) of attn_bwd: each [len(rows), H, d]."""
    H, dqk = q.shape[1], q.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    dk = np.zeros((len(rows), H, dqk), dtype=np.float64)
    dv = np.zeros((len(rows), H, v.shape[2]), dtype=np.float64)
    for n, j in enumerate(rows):
        _, _, hi = _row_seq(offsets, j)
        qs = slice(j, hi)
        for h in range(H):
            qq = np.asarray(q[qs, h], np.float64)
            s, _ = _seq_scores(qq, np.asarray(k[j:j + 1, h], np.float64), ts[qs], ts[j:j + 1],
                               np.asarray(w[h], np.float64), num_buckets, alpha)
            s = s[:, 0]
            dd = np.asarray(dout[qs, h], np.float64)
            dp = dd @ np.asarray(v[j, h], np.float64)
            g = alpha * dp * silu_grad(s)
            dv[n, h] = silu(s) @ dd
            dk[n, h] = g @ qq
    return dk, dv


# --------------------------------------------------------------------------
# 6. Target-aware attention for scoring candidates ([HSTU] App. H, M-FALCON)
#
# A sequence of n rows ends with m candidate rows after n - m history rows.
# Candidates attend to the history and must not attend to one another (App. H,
# batched inference), so one pass over history plus candidates gives each
# candidate the result of its own pass over history plus itself.  Reading:
# a candidate attends to itself (the pages do not say; the self term is what
# its own causal pass over history plus itself would contain).  With cached
# history K and V (App. H, caching) only the candidates' rows are queried.
# --------------------------------------------------------------------------

def target_mask(n: int, num_targets: int) -> np.ndarray:
    """Visibility [n, n] of key j to query i: causal, and a key among the last
    num_targets rows is visible only to itself."""
    hist = n - num_targets
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & ((j < hist) | (j == i))


def attn_fwd_targets(q, k, v, offsets, num_targets, ts, w, num_buckets) -> np.ndarray:
    """Forward over all rows with the target-aware mask; num_targets: [B]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w = np.asarray(w, np.float64)
    ts = np.asarray(ts, np.int64)
    T, H, dqk = q.shape
    alpha = 1.0 / math.sqrt(dqk)
    out = np.zeros((T, H, v.shape[2]), dtype=np.float64)
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi <= lo:
            continue
        mask = target_mask(hi - lo, int(num_targets[b]))
        for h in range(H):
            s, _ = _seq_scores(q[lo:hi, h], k[lo:hi, h], ts[lo:hi], ts[lo:hi], w[h], num_buckets, alpha)
            out[lo:hi, h] = np.where(mask, silu(s), 0.0) @ v[lo:hi, h]
    return out


def target_rows(offsets, num_targets) -> np.ndarray:
    """Global rows of the candidates, sequence by sequence."""
    rows = []
    for b in range(len(offsets) - 1):
        hi = int(offsets[b + 1])
        rows.extend(range(hi - int(num_targets[b]), hi))
    return np.asarray(rows, dtype=np.int64)


def attn_fwd_cached(q_targets, k, v, offsets, num_targets, ts, w, num_buckets) -> np.ndarray:
    """Candidates only, against cached history: q_targets [sum m_b, H, d_qk]
    holds the candidate rows in sequence order; k, v, ts cover all rows.
    Each candidate is its own pass over the history and itself."""
    q_targets = np.asarray(q_targets, np.float64)
    H, dqk = q_targets.shape[1], q_targets.shape[2]
    alpha = 1.0 / math.sqrt(dqk)
    rows = target_rows(offsets, num_targets)
    out = np.zeros((len(rows), H, v.shape[2]), dtype=np.float64)
    for n, i in enumerate(rows):
        b, lo, hi = _row_seq(offsets, int(i))
        hist = hi - int(num_targets[b])
        keys = np.concatenate([np.arange(lo, hist), [i]])
        for h in range(H):
            s, _ = _seq_scores(q_targets[n:n + 1, h], np.asarray(k[keys, h], np.float64),
                               ts[i:i + 1], np.asarray(ts)[keys], np.asarray(w[h], np.float64), num_buckets, alpha)
            out[n, h] = silu(s)[0] @ np.asarray(v[keys, h], np.float64)
    return out
