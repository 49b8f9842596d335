/*
 * hstu.h — C ABI of the MI355X (gfx950) jagged HSTU attention library.
 *
 * The operation (Scaling Generative Recommendations with Context Parallelism on
 * Hierarchical Sequential Transducers, §2.1, HSTUAttention equation):
 *
 *     O = Mask( SiLU( (Q Kᵀ + Bias) / sqrt(d_qk) ) ) V
 *
 * over jagged sequences packed token-major with int64 offsets (same paper, §2.2
 * "Jagged Tensors": values plus offsets plus max_lengths).  Mask is causal
 * (key position <= query position, diagonal included) within each sequence.
 * There is no softmax: the SiLU weights are used as they are.
 *
 * Bias (same paper, §2.1, timestamp-bias paragraph): for query i and key j of
 * one sequence, Δ = ts[i] - ts[j]; bucket = #{k in [1, NB) : |Δ| >= E_k} with
 * integer edges E_k = ceil(2^(32 k / NB)), i.e. NB equal-width bins of log2|Δ|
 * over [0, 32) (|Δ| <= 1 falls in bucket 0, |Δ| >= 2^32 in bucket NB-1);
 * Bias = ts_weights[head, bucket].  The bias is inside the division by
 * sqrt(d_qk), as the equation is set.
 *
 * Context-parallel share (same paper, §2.3, load-balanced mini-chunks): with
 * cp_size = C > 1 and cp_rank = r, every sequence of length L is cut into 2C
 * mini-chunks, chunk k being positions [floor(kL/2C), floor((k+1)L/2C)), and the
 * rank holds chunks r and 2C-1-r.  Its query rows keep their global positions
 * and global timestamps and attend to the causal key prefix of the full
 * sequence (K, V and ts are passed whole).
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless marked "host".  Tensors are dense,
 *     row-major, 16-byte aligned.  Jagged tensors are [rows, H, d].
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the device with the host.  Host metadata
 *     (max_seq_len, totals) comes from the caller.
 *   - The caller owns all memory.  The library allocates no device memory and
 *     keeps no state between calls except lazily loaded code objects and cached
 *     device attributes (thread-safe).  Scratch memory is the caller's
 *     `workspace` of at least hstu_workspace_size() bytes; it may be reused as
 *     soon as the call's work on `stream` has finished.
 *   - Outputs are overwritten, never accumulated into.
 *   - Argument errors are detected on the host before anything is launched:
 *     the call returns a non-zero hstu_status_t and hstu_last_error() gives a
 *     message.  Device-side data contracts (offsets non-decreasing with
 *     offsets[0] = 0 and offsets[B] = total_kv, every length <= max_seq_len,
 *     sum of squared lengths <= sum_sq_len when stated, |ts| < 2^62) are the
 *     caller's.
 *   - HSTU_VALIDATE: when this environment variable is set to anything but ""
 *     or "0", every call that takes offsets first checks that contract (all
 *     but the timestamp bound, plus the query row count implied for a CP
 *     share or a candidates-only pass) on the device, waits for the answer
 *     (one host synchronisation, so not for use under stream capture) and
 *     returns HSTU_EINVAL, naming what is broken, before launching anything
 *     else.  Off by default: the calls then never synchronise.
 *   - HSTU_LOG: when set to anything but "" or "0" (read once per process),
 *     every entry point that validates or launches work writes one line to
 *     stderr: its name, the problem's sizes when it takes a problem, and the
 *     status it returns with hstu_last_error's message when that is not
 *     HSTU_OK.  Logging adds no synchronisation.
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HSTU_BF16 = 0, HSTU_FP32 = 1 } hstu_dtype_t;

/* Problem flags (hstu_problem_t.flags). */
enum {
  /* Backward keeps to the memory-efficient form of the HSTU paper's App. F.3
   * (Actions Speak Louder than Words): nothing of the size of the attention
   * matrix is stored; the query-major pass recomputes the score gradient
   * instead of reading it from the workspace.  Smaller workspace, slower. */
  HSTU_FLAG_RECOMPUTE_BWD = 1,
  /* One schedule per training step: the forward and the backward of one step
   * share one workspace of hstu_workspace_size(p, 1) bytes (both calls pass
   * this flag, the same problem, the same offsets and that workspace, on one
   * stream, forward first).  The forward then builds the work lists of both
   * passes and the backward launches no scheduler of its own.  Between the
   * two calls the caller must not change offsets, the workspace or the
   * problem; a backward without its forward reads stale lists. */
  HSTU_FLAG_SHARED_SCHEDULE = 2
};

typedef enum {
  HSTU_OK = 0,
  HSTU_EINVAL = 1,        /* bad argument (null pointer, bad size, bad rank) */
  HSTU_EUNSUPPORTED = 2,  /* valid but not built: head dim, bucket count     */
  HSTU_EWORKSPACE = 3,    /* workspace missing or smaller than required      */
  HSTU_EHIP = 4           /* a HIP runtime call or kernel launch failed      */
} hstu_status_t;

/* Problem description shared by the attention calls. */
typedef struct {
  int32_t dtype;        /* hstu_dtype_t of q, k, v, out, dout, ts_weights, dq, dk, dv */
  int32_t flags;        /* HSTU_FLAG_* bits (RECOMPUTE_BWD, SHARED_SCHEDULE); others 0 */
  int64_t num_seqs;     /* B >= 0 */
  int64_t num_heads;    /* H >= 1 */
  int64_t d_qk;         /* Q/K head width; supported: 32, 64, 128 */
  int64_t d_v;          /* V head width; must equal d_qk (the kernels assume it) */
  int64_t num_buckets;  /* NB in [1, 512] */
  int64_t max_seq_len;  /* host copy of max_b (offsets[b+1] - offsets[b]) (the full
                           global length when cp_size > 1); an upper bound is fine */
  int64_t total_kv;     /* T = offsets[B]: rows of k, v, ts (and dk, dv) */
  int64_t total_q;      /* rows of q, out, dout, dq: T when cp_size == 1, else the
                           rank's row count sum_b (|chunk r| + |chunk 2C-1-r|) */
  int64_t cp_size;      /* C >= 1 (1 = whole sequences) */
  int64_t cp_rank;      /* r in [0, C) */
  int64_t sum_sq_len;   /* host copy of sum_b (offsets[b+1] - offsets[b])^2, or an upper
                           bound; 0 = not stated.  Only sizes the backward's stored
                           score gradient more tightly than max_seq_len alone can. */
} hstu_problem_t;

/* Bytes of workspace needed by hstu_jagged_attn_fwd (backward = 0) or
 * hstu_jagged_attn_bwd (backward = 1).  Returns 0 if the problem is invalid
 * (hstu_last_error() then says why).  For a forward, total_q may be smaller
 * than total_kv with cp_size 1 (the candidates-only pass).  Computed from the
 * problem's host metadata alone.  Besides the work lists it holds, for
 * problems with fewer than 1024 (128-row query tile, head) items and
 * max_seq_len > 1024, room for fp32 partial sums: there the library may split
 * the key range of long query tiles over several work items to fill the GPU
 * (the parts are summed in a fixed order, so results stay deterministic). */
size_t hstu_workspace_size(const hstu_problem_t* p, int backward);

/* Forward.  HSTUAttention equation (CP paper §2.1) on jagged inputs.
 *   q        [total_q, H, d_qk]  (cp_size > 1: the rank's rows, chunk r then
 *                                 chunk 2C-1-r per sequence, sequence-major —
 *                                 exactly the rank-r slice of hstu_cp_reorder)
 *   k        [total_kv, H, d_qk]
 *   v        [total_kv, H, d_v]
 *   offsets  int64 [B+1], global sequence offsets into k, v, ts
 *   timestamps int64 [total_kv], per-token timestamps (global)
 *   ts_weights [H, NB], bucket weights (dtype of q)
 *   out      [total_q, H, d_v] (written)
 *   workspace, workspace_bytes: scratch, >= hstu_workspace_size(p, 0)
 * Arithmetic: bf16 operands with fp32 accumulation (bf16), or fp32 throughout. */
int hstu_jagged_attn_fwd(const hstu_problem_t* p, const void* q, const void* k,
                         const void* v, const int64_t* offsets,
                         const int64_t* timestamps, const void* ts_weights,
                         void* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Forward for scoring candidates (Actions Speak Louder than Words, App. H,
 * M-FALCON: a micro-batch of candidates appended to a user's history attends
 * to the history but not to other candidates, so one pass scores the whole
 * micro-batch; with cached history K and V only the candidates are queried).
 *   num_targets int64 [B] (device): the last num_targets[b] rows of sequence
 *            b are candidates (values outside [0, its length] are clamped to
 *            it).  Key j is visible to query i iff j <= i and (j is a history
 *            row or j == i).
 *   q_targets_only = 0: q and out cover all total_kv rows (total_q must equal
 *            total_kv); history rows attend causally as in hstu_jagged_attn_fwd.
 *   q_targets_only = 1: q and out hold only the candidate rows, sequence by
 *            sequence (total_q = sum of num_targets: host metadata, like
 *            max_seq_len); k, v and timestamps cover all rows (the cached
 *            history and the candidates).
 * Requires cp_size == 1 (else HSTU_EUNSUPPORTED).  Other arguments, the
 * workspace (hstu_workspace_size(p, 0)) and the errors are as for
 * hstu_jagged_attn_fwd.  Forward only.  A candidate row gets the same bits
 * from both forms unless one of them splits the key range of the row's
 * query tile (see hstu_workspace_size); then they agree to rounding. */
int hstu_jagged_attn_fwd_targets(const hstu_problem_t* p, const void* q,
                                 const void* k, const void* v,
                                 const int64_t* offsets,
                                 const int64_t* num_targets, int q_targets_only,
                                 const int64_t* timestamps,
                                 const void* ts_weights, void* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Backward of hstu_jagged_attn_fwd for upstream gradient dout [total_q, H, d_v].
 * Writes dq [total_q, H, d_qk], dk [total_kv, H, d_qk], dv [total_kv, H, d_v]
 * (all in the input dtype, accumulated in fp32) and d_ts_weights [H, NB] (fp32).
 * With cp_size > 1, dk, dv and d_ts_weights are this rank's partial sums (zero
 * rows for keys no local query reaches); summing them over the C ranks gives
 * the gradients of the unsharded problem.  Nothing is normalised, so no
 * forward statistics are needed: the score tile is recomputed.  With bf16
 * and d_qk >= 64 the key-major pass also stores the score gradient G = dS
 * (bf16, one 64-key x 128-query block per causal tile pair, H * sum_b n_b
 * (n_b + 1) blocks of 16 KiB, n_b = ceil(L_b / 128)) in the workspace and the
 * query-major pass computes dQ = G K from it (unless p->flags has
 * HSTU_FLAG_RECOMPUTE_BWD; with cp_size > 1 only when every boundary of this
 * rank's two chunks, other than a sequence's end, is a multiple of 128 rows,
 * which the library checks on the device: otherwise G is recomputed);
 * hstu_workspace_size(p, 1) then includes room for H (N + 1)
 * (ceil(total_kv / 128) + B) blocks, N = ceil(max_seq_len / 128), or, when
 * p->sum_sq_len is stated and gives fewer, H ceil((sum_sq_len + 382 total_kv
 * + 32385 B) / 16384) blocks, unless that passes 16 GiB, in which case dQ
 * recomputes G instead.  Here max_seq_len must bound every sequence length and
 * sum_sq_len (when stated) the sum of squared lengths (blocks beyond the room
 * are dropped, not written out of bounds; HSTU_VALIDATE checks both).
 * d_ts_weights is written by the last kernel of the call (its sums are kept
 * in the workspace until then). */
int hstu_jagged_attn_bwd(const hstu_problem_t* p, const void* dout, const void* q,
                         const void* k, const void* v, const int64_t* offsets,
                         const int64_t* timestamps, const void* ts_weights,
                         void* dq, void* dk, void* dv, float* d_ts_weights,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Forward that allocates nothing, for callers that cannot allocate device
 * memory or call hipMalloc: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same operation, arguments (minus the
 * workspace), layout and errors as hstu_jagged_attn_fwd; the scratch it needs
 * (work lists, counters, bucket tables, split partial sums) lives in a
 * library-owned device array of hstu_noalloc_scratch_bytes() bytes (16 MiB)
 * that each GPU holds from the first call until the process ends.  Problems
 * whose work lists do not fit it return HSTU_EWORKSPACE before any launch
 * (about 500k query tiles of 128 rows); when the partial sums of split key
 * walks do not fit, long query tiles are walked in one item instead (same
 * result up to the order of the fp32 sums).  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (several streams, several
 * host threads) race and must be serialised by the caller.  No call to
 * hipMalloc, hipFree or hipMemset is made; the scheduler kernel rewrites all
 * the state a call reads. */
int hstu_jagged_attn_fwd_noalloc(const hstu_problem_t* p, const void* q,
                                 const void* k, const void* v,
                                 const int64_t* offsets,
                                 const int64_t* timestamps,
                                 const void* ts_weights, void* out,
                                 void* stream);

/* Bytes of the no-allocation forward's per-GPU scratch array. */
size_t hstu_noalloc_scratch_bytes(void);

/* Load-balanced chunk-pair reorder (CP paper §2.3, memory-reordering shuffle).
 * A pure row permutation of `in` [total_rows, row_bytes] into `out` (same size,
 * must not overlap `in`).  inverse = 0: sequence-major -> rank-major, i.e. for
 * r in 0..C-1, for b in 0..B-1: rows of mini-chunk r then of mini-chunk 2C-1-r
 * of sequence b.  inverse = 1: the opposite direction.  Bit-exact for any
 * row_bytes (the bytes are copied, not interpreted); rows are copied with the
 * widest of 16/8/4/1-byte accesses that row_bytes and the pointers allow.
 * out_offsets (device, may be NULL): receives the int64 [C*B + 1] offsets of
 * the rank-major segments (segment r*B + b = rank r's rows of sequence b),
 * whichever the direction.  offsets: int64 [B+1] sequence offsets of the
 * sequence-major layout; total_rows = offsets[B] < 2^42 (else
 * HSTU_EUNSUPPORTED); every sequence length must be <= max_seq_len (it sizes
 * the grid; a longer sequence is copied only in part). */
int hstu_cp_reorder(const void* in, void* out, int64_t row_bytes,
                    const int64_t* offsets, int64_t num_seqs, int64_t total_rows,
                    int64_t max_seq_len, int64_t cp_size, int inverse,
                    int64_t* out_offsets, void* stream);

/* Stochastic Length (Actions Speak Louder than Words, §3.2 and §4.2: long
 * histories are sparsified by keeping a subsequence; at alpha = 1.6 a
 * length-4096 history becomes length 776 most of the time; App. E: the
 * subsequence is chosen by recency or at random, among other criteria).
 * Selection only; hstu_gather_rows then moves any tensor's rows.
 *   offsets      int64 [B+1], sequence offsets of the input rows
 *   alpha        in (0, 64): a sequence of length n is cut to
 *                L = floor(n^(alpha/2)) rows (computed in double precision,
 *                an exact integer power kept exact), unless
 *   seq_uniform  float [B], one draw in [0, 1) per sequence: kept whole when
 *                seq_uniform[b] < n^(alpha-2) (probability n^(alpha-2)), or
 *                when L >= n
 *   token_keys   uint32 [total_rows] random keys (device), or NULL.  Keys
 *                given: the L rows with the smallest keys are kept (equal
 *                keys in position order); NULL: the last L rows (recency).
 *   out_offsets  int64 [B+1] (written): offsets of the kept rows
 *   out_index    int64 [total_rows] (written for the first out_offsets[B]
 *                entries): the input row of every output row; the kept rows
 *                of a sequence stay in their original order.
 * The output row count out_offsets[B] stays on the device (no host sync);
 * total_rows bounds it.  Two launches on `stream`. */
int hstu_sl_select(const int64_t* offsets, int64_t num_seqs, int64_t total_rows,
                   int64_t max_seq_len, double alpha, const float* seq_uniform,
                   const uint32_t* token_keys, int64_t* out_offsets,
                   int64_t* out_index, void* stream);

/* Row gather: out[i] = in[index[i]] for i < min(*count, max_rows), rows of
 * row_bytes bytes copied unchanged (bit-exact, widest of 16/8/4/1-byte
 * accesses that row_bytes and both pointers allow).  count is a device
 * pointer (e.g. out_offsets + B of hstu_sl_select), so the call needs no host
 * synchronisation; max_rows bounds the launch.  index entries must be valid
 * rows of `in` (the caller's contract, as hstu_sl_select's output is). */
int hstu_gather_rows(const void* in, void* out, int64_t row_bytes,
                     const int64_t* index, const int64_t* count,
                     int64_t max_rows, void* stream);

/* HSTU layer steps either side of the attention (Actions Speak Louder than
 * Words, §3: pointwise projection, spatial aggregation, pointwise
 * transformation; the interaction is Norm(A(X)V(X)) ⊙ U(X)).  bf16 in and out,
 * fp32 accumulation.  The pages name the steps but not their exact form; the
 * forms built are: the projection is one linear map without bias then SiLU,
 * split in the order U, V, Q, K; Norm is layer normalisation over a row's
 * H d_v attention outputs without learned scale or shift.
 *
 * Projection: [U V Q K] = SiLU(x wᵀ).
 *   x  [total_rows, d_model]; d_model a multiple of 64
 *   w  [H (2 d_v + 2 d_qk), d_model] (a linear layer's weight layout)
 *   u, v  [total_rows, H, d_v] (written); q, k [total_rows, H, d_qk] (written),
 *   ready for hstu_jagged_attn_fwd.  H d_v and H d_qk must be multiples of 128
 *   (else HSTU_EUNSUPPORTED). */
int hstu_layer_projection(const void* x, const void* w, int64_t total_rows,
                          int64_t d_model, int64_t num_heads, int64_t d_qk,
                          int64_t d_v, void* u, void* v, void* q, void* k,
                          void* stream);

/* Pointwise transformation: y = Norm(o) ⊙ u, row by row.
 *   o  [total_rows, width] (the attention output [T, H, d_v], width = H d_v)
 *   u  [total_rows, width]; y [total_rows, width] (written)
 *   Norm(r) = (r - mean(r)) / sqrt(var(r) + eps), biased variance, statistics
 *   in fp32; width a multiple of 8, at most 4096. */
int hstu_layer_norm_gate(const void* o, const void* u, void* y,
                         int64_t total_rows, int64_t width, double eps,
                         void* stream);

/* Host helper: the integer bucket edges the kernels use.  Writes NB+1 uint32
 * values to host memory edges_out: edges_out[0] = 0, edges_out[k] = E_k =
 * ceil(2^(32k/NB)) for 1 <= k < NB, edges_out[NB] = 0xFFFFFFFF (sentinel). */
int hstu_bucket_edges(int64_t num_buckets, uint32_t* edges_out);

/* Message for the last non-OK status returned on the calling thread. */
const char* hstu_last_error(void);

/* Optional per-kernel timing, for profiling.  While enabled, every kernel this
 * library launches is bracketed by two HIP events recorded on the launch
 * stream (so the measured interval is that kernel's execution on its stream).
 * hstu_timing_read waits for the recorded events (host-blocking) and returns
 * the milliseconds and launch count accumulated for one kernel since the last
 * hstu_timing_reset.  Off by default; the events are created and destroyed by
 * the library (no device memory).  Not for use inside a stream capture. */
typedef enum {
  HSTU_KERNEL_SCHED = 0,    /* tile scheduler (one workgroup) */
  HSTU_KERNEL_FWD = 1,      /* forward attention */
  HSTU_KERNEL_BWD_KV = 2,   /* backward, key-major pass: dK, dV, d(ts_weights) */
  HSTU_KERNEL_BWD_Q = 3,    /* backward, query-major pass: dQ */
  HSTU_KERNEL_REORDER = 4,  /* chunk-pair reorder */
  HSTU_KERNEL_REDUCE = 5,   /* sum of the parts of split query tiles (forward or dQ) */
  HSTU_KERNEL_SL = 6,       /* Stochastic Length selection (lengths, then rows) */
  HSTU_KERNEL_GATHER = 7,   /* row gather */
  HSTU_KERNEL_PROJ = 8,     /* layer projection GEMM with SiLU */
  HSTU_KERNEL_NORM_GATE = 9,  /* layer norm-gate */
  HSTU_KERNEL_COUNT = 10
} hstu_kernel_t;
int hstu_timing_enable(int on);
int hstu_timing_reset(void);
int hstu_timing_read(int kernel, double* total_ms /* host */, int64_t* launches /* host */);

/* Library version: major * 10000 + minor * 100 + patch. */
int hstu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H */
