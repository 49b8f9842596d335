// Jagged HSTU attention kernels for gfx950: forward, dK/dV/d(ts_weights) pass
// and dQ pass.  All three are persistent: every workgroup pops work items
// (tile x head) from a descending-cost list built by the scheduler kernel.
//
// The operation (Scaling Generative Recommendations with Context Parallelism on
// HSTU, §2.1, HSTUAttention equation and timestamp-bias paragraph):
//   s_ij = alpha * (q_i . k_j + w[h, bucket(ts_i - ts_j)]),  alpha = 1/sqrt(d)
//   a_ij = SiLU(s_ij) * [pos_j <= pos_i]
//   O_i  = sum_j a_ij v_j
// Backward: dP = dO Vᵀ, G = alpha * dP * SiLU'(s) * mask, dV = aᵀ dO,
// dK = Gᵀ Q, dQ = G K, dW[h, b] = sum of G over pairs in bucket b.
//
// Every lane owns one row for the whole item (a query in the forward and dQ
// passes, a key in the dK/dV pass), so the timestamp of its row, its causal
// limit and its bias plan (epilogue.h) are per-lane scalars.  The other side
// streams through double-buffered, swizzled LDS tiles (swtile.h) filled with
// direct-to-LDS loads one tile ahead; one barrier per tile.
#include "attn.h"
#include "epilogue.h"
#include "swtile.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int BM = 128;        // query rows per forward / dQ item (32 per wave)
constexpr int BN = 64;         // keys per tile in the forward / dQ loops
constexpr int BK = 128;        // keys per dK/dV item (32 per wave)
constexpr int BQ = 64;         // query rows per step of the dK/dV loop
static_assert(BQ == BN, "the dK/dV step tiles share the key-tile shape");

// d(ts_weights) bins are kept in kDwCopies interleaved copies (lane l adds to
// copy l % kDwCopies) so that lanes of one instruction that hit the same bucket
// mostly hit different addresses; the copies are summed at flush time.
constexpr int kDwCopies = 8;

struct alignas(16) Tables {
  float w[kMaxBuckets];                         // alpha * ts_weights[h, :]
  u32x2 ep[kMaxBuckets];                        // bucket edge pairs (E[k], E[k+1])
  float dw[kDwCopies][kMaxBuckets + 1];         // per-item d(ts_weights) bins (backward)
  int item;
};

struct alignas(16) TablesFwd {
  float w[kMaxBuckets];
  u32x2 ep[kMaxBuckets];
  int item;
};

template <typename TB>
__device__ __forceinline__ void load_edges(TB& t, const AttnParams& p, int tid) {
  for (int i = tid; i < p.NB; i += kThreads) t.ep[i] = u32x2{p.edges[i], p.edges[i + 1]};
}

template <typename T, typename TB>
__device__ __forceinline__ void load_wtab(TB& t, const AttnParams& p, int h, int tid) {
  const T* W = static_cast<const T*>(p.w) + (int64_t)h * p.NB;
  for (int i = tid; i < p.NB; i += kThreads) t.w[i] = p.alpha * to_f32<T>(W[i]);
}

template <typename TB>
__device__ __forceinline__ int pop_item(TB& t, int* counter, int tid) {
  __syncthreads();
  if (tid == 0) t.item = atomicAdd(counter, 1);
  __syncthreads();
  return t.item;
}

// Rank-local query segments of sequence b: (local row start, first position,
// length).  cp_size == 1: one segment covering the sequence.
struct Seg {
  int64_t row0;
  int pos0;
  int len;
};

__device__ __forceinline__ int q_segments(const AttnParams& p, int b, Seg* seg) {
  const int64_t o0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - o0);
  if (p.cp_size == 1) {
    seg[0] = Seg{o0, 0, L};
    return 1;
  }
  const int nch = 2 * p.cp_size;
  const int c0 = p.cp_rank, c1 = nch - 1 - p.cp_rank;
  const int a0 = (int)((int64_t)c0 * L / nch), a1 = (int)((int64_t)(c0 + 1) * L / nch);
  const int b0 = (int)((int64_t)c1 * L / nch), b1 = (int)((int64_t)(c1 + 1) * L / nch);
  const int64_t lo = p.local_off[b];
  seg[0] = Seg{lo, a0, a1 - a0};
  seg[1] = Seg{lo + (a1 - a0), b0, b1 - b0};
  return 2;
}

// Steps of BQ query rows, over the (at most two) segments, from position
// `start` on.  Segments are held in scalar fields (selected by index) so that
// the iterator stays in registers.
struct StepIter {
  int64_t r0, r1;  // local row of each segment's first position
  int p0, p1;      // first position of each segment
  int e0, e1;      // end position of each segment
  int nseg;
  int start;
  int si;
  int q0;
  __device__ __forceinline__ int seg_pos(int i) const { return i == 0 ? p0 : p1; }
  __device__ __forceinline__ int seg_end(int i) const { return i == 0 ? e0 : e1; }
  __device__ __forceinline__ void norm() {
    if (si == 0 && q0 >= e0) {
      si = 1;
      q0 = max(p1, start);
    }
    if (si == 1 && (nseg < 2 || q0 >= e1)) si = 2;
  }
  __device__ __forceinline__ void init(const AttnParams& p, int b, int start_pos) {
    Seg seg[2];
    nseg = q_segments(p, b, seg);
    r0 = seg[0].row0;
    p0 = seg[0].pos0;
    e0 = seg[0].pos0 + seg[0].len;
    r1 = nseg > 1 ? seg[1].row0 : 0;
    p1 = nseg > 1 ? seg[1].pos0 : 0;
    e1 = nseg > 1 ? seg[1].pos0 + seg[1].len : 0;
    start = start_pos;
    si = 0;
    q0 = max(p0, start);
    norm();
  }
  __device__ __forceinline__ bool valid() const { return si < nseg; }
  __device__ __forceinline__ int nq() const { return min(BQ, seg_end(si) - q0); }
  __device__ __forceinline__ int64_t lrow() const { return (si == 0 ? r0 : r1) + (q0 - seg_pos(si)); }
  __device__ __forceinline__ void next() {
    q0 += BQ;
    norm();
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// Forward.  One item = (query tile of 128 rows, head).  Wave w owns query rows
// 32w..32w+31 of the tile; lane (r32, g) owns query row 32w + r32: the score
// tile is computed transposed, Sᵀ = K Qᵀ, so every accumulator value of a lane
// belongs to its own query, and the output is Oᵀ = Vᵀ Pᵀ with P taken straight
// from the Sᵀ accumulators (V read with transpose reads).
// ---------------------------------------------------------------------------
template <typename T, int D> struct alignas(16) KvSmem {
  T k[2][BN * D];
  T v[2][BN * D];
  TsTile<BN> ts[2];
};

template <typename T, int D>
__device__ __forceinline__ void issue_kv(KvSmem<T, D>& sm, int buf, const T* Kh, const T* Vh, int64_t ld, int key0,
                                         int nvalid, int tid) {
  tile_load_async<T, D, BN, kThreads>(sm.k[buf], Kh + key0 * ld, ld, nvalid, tid);
  tile_load_async<T, D, BN, kThreads>(sm.v[buf], Vh + key0 * ld, ld, nvalid, tid);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ KvSmem<T, D> sm;
  __shared__ TablesFwd tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  LaneOffsets<D> lo;
  if constexpr (kBf16) lo.init(lane);
  const int H = p.H, NB = p.NB;
  const float nb32 = NB * (1.0f / 32.0f);
  const float alpha = p.alpha;
  const int64_t ld = (int64_t)H * D;
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  T* O = static_cast<T*>(p.out);
  load_edges(tb, p, tid);
  const int n_work = p.ctr[kCtrQTiles] * H;

  for (;;) {
    const int w = pop_item(tb, p.ctr + kCtrQNext, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.qitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int qi = wave * 32 + r32;
    const bool qvalid = qi < it.n;
    const int qpos = it.pos0 + qi;
    const int64_t qrow = (int64_t)it.row0 + qi;
    const int64_t tsq = qvalid ? p.ts[seq0 + qpos] : 0;
    op_t qop[D / M::kK];
#pragma unroll
    for (int kk = 0; kk < D / M::kK; ++kk) {
      qop[kk] = op_t{};
      if (qvalid) qop[kk] = M::load(Q + qrow * ld + h * D + kk * M::kK + g * M::kEpl);
    }
    load_wtab<T>(tb, p, h, tid);
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};

    const int kv_len = it.pos0 + it.n;
    const int n_kt = (kv_len + BN - 1) / BN;
    const int wave_qmin = it.pos0 + wave * 32;
    const T* Kh = K + seq0 * ld + h * D;
    const T* Vh = V + seq0 * ld + h * D;
    int64_t tsv = 0;
    issue_kv<T, D>(sm, 0, Kh, Vh, ld, 0, min(BN, kv_len), tid);
    if (wave == 0) tsv = p.ts[seq0 + min(lane, kv_len - 1)];
    if (wave == 0) ts_tile_fill<BN, false>(sm.ts[0], tsv, min(BN, kv_len), lane);
    wait_loads();
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
      const int cur = kt & 1;
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      const bool more = kt + 1 < n_kt;
      if (more) {
        const int nk0 = key0 + BN, nnv = min(BN, kv_len - nk0);
        issue_kv<T, D>(sm, cur ^ 1, Kh, Vh, ld, nk0, nnv, tid);
        if (wave == 0) tsv = p.ts[seq0 + nk0 + min(lane, nnv - 1)];
      }
      const T* kt_ = sm.k[cur];
      const T* vt_ = sm.v[cur];
      const TsTile<BN>& ts = sm.ts[cur];

      const int lim = min(nvalid - 1, qpos - key0);
      const bool any = qvalid && lim >= 0;
      int64_t tmin = 0, tmax = 0;
      ts_tile_range<BN, false>(ts, 0, any ? lim : 0, &tmin, &tmax);
      const LaneBias lb = lane_bias<+1>(tsq, tmin, tmax, any, ts.base, ts.wide, tb.w, tb.ep, NB, nb32);
      const int mode = wave_mode(lb.n);
      int32_t tsr_rel = 0;
      const bool fast32 = mode == kModeExact && wave_fast32(tsq, ts.base, ts.wide, &tsr_rel);
      const bool diag = key0 + BN - 1 > wave_qmin;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) {
        f32x16 s;
        if constexpr (kBf16)
          s = tile_mma_rows_o<D>(reinterpret_cast<const char*>(kt_), lo, blk, qop);
        else
          s = tile_mma_rows<T, D>(kt_, blk * 32 + r32, qop, g);
        float cb[16];
        int bsel[16];
        block_bias<+1, BN>(cb, bsel, mode, lb, tsq, tsr_rel, fast32, ts, blk, g, tb.w, tb.ep, NB, nb32);
        float pv[16];
        if (diag) {
          const int lim_row = qpos - key0 - blk * 32;  // values with row > lim_row are masked
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = fmaf(s[i], alpha, cb[i]);
            const float a = x * fast_sigmoid(x);
            pv[i] = acc_row(i, g) > lim_row ? 0.0f : a;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = fmaf(s[i], alpha, cb[i]);
            pv[i] = x * fast_sigmoid(x);
          }
        }
        if constexpr (kBf16)
          tile_contract_block_o<D>(oacc, reinterpret_cast<const char*>(vt_), lo, pv, blk);
        else
          tile_contract_block<T, D>(oacc, vt_, pv, blk, lane);
      }
      if (more && wave == 0) ts_tile_fill<BN, false>(sm.ts[cur ^ 1], tsv, min(BN, kv_len - key0 - BN), lane);
      wait_loads();
      __syncthreads();
    }
    if (qvalid) store_row_from_acc<T, D>(O + qrow * ld + h * D, oacc, g);
  }
}

// ---------------------------------------------------------------------------
// Backward, key-major pass: dK, dV and d(ts_weights).  One item = (key tile of
// 128 keys, head); lane (r32, g) of wave w owns key 32w + r32.  For each step of
// 64 query rows it computes S = Q Kᵀ and dP = dO Vᵀ (so the lane's values all
// belong to its own key), then dVᵀ += dOᵀ P and dKᵀ += Qᵀ G, reading Q and dO
// transposed from the same tiles.  Query rows past the end of a step replicate
// the last row; their P and G are masked to zero.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_kv_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ KvSmem<T, D> sm;  // k: query rows, v: dO rows
  __shared__ Tables tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  LaneOffsets<D> lo;
  if constexpr (kBf16) lo.init(lane);
  const int H = p.H, NB = p.NB;
  const float nb32 = NB * (1.0f / 32.0f);
  const float alpha = p.alpha;
  const int64_t ld = (int64_t)H * D;
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* dO = static_cast<const T*>(p.dout);
  T* dK = static_cast<T*>(p.dk);
  T* dV = static_cast<T*>(p.dv);
  load_edges(tb, p, tid);
  const int n_work = p.ctr[kCtrKTiles] * H;

  for (;;) {
    const int w = pop_item(tb, p.ctr + kCtrKNext, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.kitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int kj = wave * 32 + r32;
    const bool kvalid = kj < it.n;
    const int kpos = it.pos0 + kj;
    const int64_t krow = (int64_t)it.row0 + kj;
    const int64_t tsk = kvalid ? p.ts[krow] : 0;
    op_t kop[D / M::kK], vop[D / M::kK];
#pragma unroll
    for (int kk = 0; kk < D / M::kK; ++kk) {
      kop[kk] = op_t{};
      vop[kk] = op_t{};
      if (kvalid) {
        kop[kk] = M::load(K + krow * ld + h * D + kk * M::kK + g * M::kEpl);
        vop[kk] = M::load(V + krow * ld + h * D + kk * M::kK + g * M::kEpl);
      }
    }
    load_wtab<T>(tb, p, h, tid);
    for (int i = tid; i < kDwCopies * (kMaxBuckets + 1); i += kThreads) (&tb.dw[0][0])[i] = 0.0f;
    float* dwl = tb.dw[lane % kDwCopies];
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      dkacc[i] = f32x16{};
      dvacc[i] = f32x16{};
    }
    const int wave_kmax = it.pos0 + wave * 32 + 31;

    int64_t tsv = 0;
    StepIter si;
    si.init(p, it.b, it.pos0);
    int cur = 0;
    if (si.valid()) {
      issue_kv<T, D>(sm, 0, Q + h * D, dO + h * D, ld, (int)si.lrow(), si.nq(), tid);
      if (wave == 0) tsv = p.ts[seq0 + si.q0 + min(lane, si.nq() - 1)];
      if (wave == 0) ts_tile_fill<BQ, true>(sm.ts[0], tsv, si.nq(), lane);
    }
    wait_loads();
    __syncthreads();
    while (si.valid()) {
      const int q0 = si.q0;
      const int nq = si.nq();
      StepIter nx = si;
      nx.next();
      if (nx.valid()) {
        issue_kv<T, D>(sm, cur ^ 1, Q + h * D, dO + h * D, ld, (int)nx.lrow(), nx.nq(), tid);
        if (wave == 0) tsv = p.ts[seq0 + nx.q0 + min(lane, nx.nq() - 1)];
      }
      const T* qt_ = sm.k[cur];
      const T* dt_ = sm.v[cur];
      const TsTile<BQ>& ts = sm.ts[cur];

      const int first = max(0, kpos - q0);
      const bool any = kvalid && first < nq;
      int64_t tmin = 0, tmax = 0;
      ts_tile_range<BQ, true>(ts, any ? first : BQ - 1, BQ - 1, &tmin, &tmax);
      const LaneBias lb = lane_bias<-1>(tsk, tmin, tmax, any, ts.base, ts.wide, tb.w, tb.ep, NB, nb32);
      const int mode = wave_mode(lb.n);
      int32_t tsr_rel = 0;
      const bool fast32 = mode == kModeExact && wave_fast32(tsk, ts.base, ts.wide, &tsr_rel);
      const bool needmask = q0 < wave_kmax || nq < BQ;
      float dwb[kMaxEdges + 1] = {0.0f, 0.0f, 0.0f, 0.0f};  // bins b_lo + k
#pragma unroll
      for (int blk = 0; blk < BQ / 32; ++blk) {
        f32x16 s, dp;
        if constexpr (kBf16) {
          s = tile_mma_rows_o<D>(reinterpret_cast<const char*>(qt_), lo, blk, kop);
          dp = tile_mma_rows_o<D>(reinterpret_cast<const char*>(dt_), lo, blk, vop);
        } else {
          s = tile_mma_rows<T, D>(qt_, blk * 32 + r32, kop, g);
          dp = tile_mma_rows<T, D>(dt_, blk * 32 + r32, vop, g);
        }
        float cb[16];
        int bsel[16];
        block_bias<-1, BQ>(cb, bsel, mode, lb, tsk, tsr_rel, fast32, ts, blk, g, tb.w, tb.ep, NB, nb32);
        float pv[16], gv[16];
        // query row qj is visible iff kpos <= q0 + qj and qj < nq
        const int lo_row = kpos - q0 - blk * 32, hi_row = nq - blk * 32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = fmaf(s[i], alpha, cb[i]);
          const float sg = fast_sigmoid(x);
          float a = x * sg;
          float gg = alpha * dp[i] * (sg * (1.0f + x * (1.0f - sg)));
          if (needmask) {
            const int r = acc_row(i, g);
            const bool vis = r >= lo_row && r < hi_row;
            a = vis ? a : 0.0f;
            gg = vis ? gg : 0.0f;
          }
          pv[i] = a;
          gv[i] = gg;
          if (mode == kModeExact) {
            if (gg != 0.0f) atomicAdd(&dwl[bsel[i]], gg);
          } else {
#pragma unroll
            for (int k = 0; k <= kMaxEdges; ++k)
              if (k <= mode) dwb[k] += bsel[i] == k ? gg : 0.0f;
          }
        }
        if constexpr (kBf16) {
          tile_contract_block_o<D>(dvacc, reinterpret_cast<const char*>(dt_), lo, pv, blk);
          tile_contract_block_o<D>(dkacc, reinterpret_cast<const char*>(qt_), lo, gv, blk);
        } else {
          tile_contract_block<T, D>(dvacc, dt_, pv, blk, lane);
          tile_contract_block<T, D>(dkacc, qt_, gv, blk, lane);
        }
      }
      if (mode != kModeExact) {
#pragma unroll
        for (int k = 0; k <= kMaxEdges; ++k)
          if (dwb[k] != 0.0f) atomicAdd(&dwl[lb.b_lo + k], dwb[k]);
      }
      if (nx.valid() && wave == 0) ts_tile_fill<BQ, true>(sm.ts[cur ^ 1], tsv, nx.nq(), lane);
      wait_loads();
      __syncthreads();
      si = nx;
      cur ^= 1;
    }
    if (kvalid) {
      store_row_from_acc<T, D>(dK + krow * ld + h * D, dkacc, g);
      store_row_from_acc<T, D>(dV + krow * ld + h * D, dvacc, g);
    }
    for (int i = tid; i < NB; i += kThreads) {
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < kDwCopies; ++c) v += tb.dw[c][i];
      if (v != 0.0f) atomicAdd(p.dw + (int64_t)h * NB + i, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major pass: dQ.  Same item list and lane ownership as the
// forward; Sᵀ = K Qᵀ and dPᵀ = V dOᵀ are recomputed and dQᵀ += Kᵀ Gᵀ (K read
// transposed from the same tile).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ KvSmem<T, D> sm;
  __shared__ TablesFwd tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  LaneOffsets<D> lo;
  if constexpr (kBf16) lo.init(lane);
  const int H = p.H, NB = p.NB;
  const float nb32 = NB * (1.0f / 32.0f);
  const float alpha = p.alpha;
  const int64_t ld = (int64_t)H * D;
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* dO = static_cast<const T*>(p.dout);
  T* dQ = static_cast<T*>(p.dq);
  load_edges(tb, p, tid);
  const int n_work = p.ctr[kCtrQTiles] * H;

  for (;;) {
    const int w = pop_item(tb, p.ctr + kCtrQNext2, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.qitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int qi = wave * 32 + r32;
    const bool qvalid = qi < it.n;
    const int qpos = it.pos0 + qi;
    const int64_t qrow = (int64_t)it.row0 + qi;
    const int64_t tsq = qvalid ? p.ts[seq0 + qpos] : 0;
    op_t qop[D / M::kK], dop[D / M::kK];
#pragma unroll
    for (int kk = 0; kk < D / M::kK; ++kk) {
      qop[kk] = op_t{};
      dop[kk] = op_t{};
      if (qvalid) {
        qop[kk] = M::load(Q + qrow * ld + h * D + kk * M::kK + g * M::kEpl);
        dop[kk] = M::load(dO + qrow * ld + h * D + kk * M::kK + g * M::kEpl);
      }
    }
    load_wtab<T>(tb, p, h, tid);
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};

    const int kv_len = it.pos0 + it.n;
    const int n_kt = (kv_len + BN - 1) / BN;
    const int wave_qmin = it.pos0 + wave * 32;
    const T* Kh = K + seq0 * ld + h * D;
    const T* Vh = V + seq0 * ld + h * D;
    int64_t tsv = 0;
    issue_kv<T, D>(sm, 0, Kh, Vh, ld, 0, min(BN, kv_len), tid);
    if (wave == 0) tsv = p.ts[seq0 + min(lane, kv_len - 1)];
    if (wave == 0) ts_tile_fill<BN, false>(sm.ts[0], tsv, min(BN, kv_len), lane);
    wait_loads();
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
      const int cur = kt & 1;
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      const bool more = kt + 1 < n_kt;
      if (more) {
        const int nk0 = key0 + BN, nnv = min(BN, kv_len - nk0);
        issue_kv<T, D>(sm, cur ^ 1, Kh, Vh, ld, nk0, nnv, tid);
        if (wave == 0) tsv = p.ts[seq0 + nk0 + min(lane, nnv - 1)];
      }
      const T* kt_ = sm.k[cur];
      const T* vt_ = sm.v[cur];
      const TsTile<BN>& ts = sm.ts[cur];

      const int lim = min(nvalid - 1, qpos - key0);
      const bool any = qvalid && lim >= 0;
      int64_t tmin = 0, tmax = 0;
      ts_tile_range<BN, false>(ts, 0, any ? lim : 0, &tmin, &tmax);
      const LaneBias lb = lane_bias<+1>(tsq, tmin, tmax, any, ts.base, ts.wide, tb.w, tb.ep, NB, nb32);
      const int mode = wave_mode(lb.n);
      int32_t tsr_rel = 0;
      const bool fast32 = mode == kModeExact && wave_fast32(tsq, ts.base, ts.wide, &tsr_rel);
      const bool diag = key0 + BN - 1 > wave_qmin;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) {
        f32x16 s, dp;
        if constexpr (kBf16) {
          s = tile_mma_rows_o<D>(reinterpret_cast<const char*>(kt_), lo, blk, qop);
          dp = tile_mma_rows_o<D>(reinterpret_cast<const char*>(vt_), lo, blk, dop);
        } else {
          s = tile_mma_rows<T, D>(kt_, blk * 32 + r32, qop, g);
          dp = tile_mma_rows<T, D>(vt_, blk * 32 + r32, dop, g);
        }
        float cb[16];
        int bsel[16];
        block_bias<+1, BN>(cb, bsel, mode, lb, tsq, tsr_rel, fast32, ts, blk, g, tb.w, tb.ep, NB, nb32);
        float gv[16];
        const int lim_row = qpos - key0 - blk * 32;  // values with row > lim_row are masked
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = fmaf(s[i], alpha, cb[i]);
          const float sg = fast_sigmoid(x);
          const float gg = alpha * dp[i] * (sg * (1.0f + x * (1.0f - sg)));
          gv[i] = (diag && acc_row(i, g) > lim_row) ? 0.0f : gg;
        }
        if constexpr (kBf16)
          tile_contract_block_o<D>(dqacc, reinterpret_cast<const char*>(kt_), lo, gv, blk);
        else
          tile_contract_block<T, D>(dqacc, kt_, gv, blk, lane);
      }
      if (more && wave == 0) ts_tile_fill<BN, false>(sm.ts[cur ^ 1], tsv, min(BN, kv_len - key0 - BN), lane);
      wait_loads();
      __syncthreads();
    }
    if (qvalid) store_row_from_acc<T, D>(dQ + qrow * ld + h * D, dqacc, g);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
template <typename K>
int grid_for(K kernel, int max_items, int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int g = cus * per_cu;
  return max(1, min(g, max_items));
}

template <typename T, int D>
hipError_t launch_all(const AttnParams& p, int which, int max_items, int cus, hipStream_t s) {
  if (which == 0) {
    auto k = fwd_kernel<T, D>;
    hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus)), dim3(kThreads), 0, s, p);
  } else if (which == 1) {
    auto k = bwd_kv_kernel<T, D>;
    hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus)), dim3(kThreads), 0, s, p);
  } else {
    auto k = bwd_q_kernel<T, D>;
    hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus)), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const AttnParams& p, int d, int which, int max_items, int cus, hipStream_t s) {
  switch (d) {
    case 32: return launch_all<T, 32>(p, which, max_items, cus, s);
    case 64: return launch_all<T, 64>(p, which, max_items, cus, s);
    case 128: return launch_all<T, 128>(p, which, max_items, cus, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_attn(const AttnParams& p, bool bf16, int d, int which, int max_items, int cus, hipStream_t s) {
  return bf16 ? launch_d<__bf16>(p, d, which, max_items, cus, s) : launch_d<float>(p, d, which, max_items, cus, s);
}

int attn_q_tile_rows() { return BM; }
int attn_k_tile_keys() { return BN; }
int attn_bwd_key_tile() { return BK; }
int attn_bwd_q_step() { return BQ; }

}  // namespace hstu
