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
#include "attn.h"
#include "tiles.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;  // 4 waves

template <typename T, int D> struct FwdCfg {
  static constexpr int BM = 128;  // query rows per item (32 per wave)
  static constexpr int BN = 64;   // keys per tile
};

template <typename T, int D, int BN> struct alignas(16) KvTiles {
  T k[BN * Pitch<T, D>::row];
  // bf16: V transposed ([d][slot]); fp32: V row-major.
  T v[sizeof(T) == 2 ? D * TPitch<BN>::col : BN * Pitch<T, D>::row];
  int64_t ts[BN];
};

struct alignas(16) Tables {
  float w[kMaxBuckets];          // alpha * ts_weights[h, :]
  uint32_t e[kMaxBuckets + 4];   // bucket edges E[0..NB]
  float dw[kMaxBuckets];         // per-item d(ts_weights) bins (backward)
  int item;
};

__device__ __forceinline__ void load_edges(Tables& t, const AttnParams& p, int tid) {
  for (int i = tid; i <= p.NB; i += kThreads) t.e[i] = p.edges[i];
}

template <typename T>
__device__ __forceinline__ void load_wtab(Tables& t, const AttnParams& p, int h, int tid) {
  const T* W = static_cast<const T*>(p.w) + (int64_t)h * p.NB;
  for (int i = tid; i < p.NB; i += kThreads) t.w[i] = p.alpha * to_f32<T>(W[i]);
}

__device__ __forceinline__ int pop_item(Tables& t, int* counter, int tid) {
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

}  // namespace

// ---------------------------------------------------------------------------
// Forward.  One item = (query tile of 128 rows, head).  Wave w owns query rows
// 32w..32w+31 of the tile; lane (r32, g) owns query row 32w + r32 throughout:
// the score tile is computed transposed, Sᵀ = K Qᵀ, so every accumulator value
// of a lane belongs to its own query row, and the output is computed as
// Oᵀ = Vᵀ Pᵀ with P taken straight from the Sᵀ accumulators.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr int BN = FwdCfg<T, D>::BN;
  __shared__ KvTiles<T, D, BN> kv;
  __shared__ Tables tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  const int H = p.H;
  const float nb32 = p.NB * (1.0f / 32.0f);
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
    for (int kt = 0; kt < n_kt; ++kt) {
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      __syncthreads();
      const int64_t krow = seq0 + key0;
      stage_rows<T, D, BN, kThreads>(kv.k, K + krow * ld + h * D, ld, nvalid, tid);
      if constexpr (sizeof(T) == 2)
        stage_rows_t<D, BN, kThreads>(kv.v, V + krow * ld + h * D, ld, nvalid, tid);
      else
        stage_rows<T, D, BN, kThreads>(kv.v, V + krow * ld + h * D, ld, nvalid, tid);
      for (int j = tid; j < BN; j += kThreads) kv.ts[j] = j < nvalid ? p.ts[krow + j] : 0;
      __syncthreads();

      float pv[BN / 32][16];
      const bool diag = key0 + BN - 1 > it.pos0;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) {
        const f32x16 s = mma_tile_rows<T, D>(kv.k, blk * 32 + r32, qop, g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = blk * 32 + acc_row(i, g);
          const int bk = bucket_of(tsq - kv.ts[kj], p.NB, nb32, tb.e);
          const float x = fmaf(s[i], p.alpha, tb.w[bk]);
          float a = x * fast_sigmoid(x);
          if (diag && key0 + kj > qpos) a = 0.0f;
          pv[blk][i] = a;
        }
      }
      mma_contract_rows<T, D, BN>(oacc, kv.v, pv, r32, g);
    }
    if (qvalid) store_row_from_acc<T, D>(O + qrow * ld + h * D, oacc, g);
  }
}

// ---------------------------------------------------------------------------
// Backward, key-major pass: dK, dV and d(ts_weights).  One item = (key tile of
// 128 keys, head); lane (r32, g) of wave w owns key 32w + r32.  For each step of
// 64 query rows it computes S = Q Kᵀ and dP = dO Vᵀ (so the lane's values all
// belong to its own key), then dVᵀ += dOᵀ P and dKᵀ += Qᵀ G.
// ---------------------------------------------------------------------------
template <typename T, int D> struct BwdKvCfg {
  static constexpr int BK = 128;  // keys per item
  static constexpr int BQ = 64;   // query rows per step
};

template <typename T, int D, int BQ> struct alignas(16) QdoTiles {
  T q[BQ * Pitch<T, D>::row];
  T dout[BQ * Pitch<T, D>::row];
  T qt[sizeof(T) == 2 ? D * TPitch<BQ>::col : 1];
  T doutt[sizeof(T) == 2 ? D * TPitch<BQ>::col : 1];
  int64_t ts[BQ];
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_kv_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr int BQ = BwdKvCfg<T, D>::BQ;
  __shared__ QdoTiles<T, D, BQ> qt;
  __shared__ Tables tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  const int H = p.H;
  const float nb32 = p.NB * (1.0f / 32.0f);
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
    for (int i = tid; i < p.NB; i += kThreads) tb.dw[i] = 0.0f;
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      dkacc[i] = f32x16{};
      dvacc[i] = f32x16{};
    }

    Seg seg[2];
    const int nseg = q_segments(p, it.b, seg);
    for (int sgi = 0; sgi < nseg; ++sgi) {
      const Seg sg = seg[sgi];
      const int segend = sg.pos0 + sg.len;
      // queries at positions >= it.pos0 can see some key of the tile
      const int start = max(sg.pos0, it.pos0);
      for (int q0 = start; q0 < segend; q0 += BQ) {
        const int nq = min(BQ, segend - q0);
        const int64_t lrow = sg.row0 + (q0 - sg.pos0);
        __syncthreads();
        stage_rows<T, D, BQ, kThreads>(qt.q, Q + lrow * ld + h * D, ld, nq, tid);
        stage_rows<T, D, BQ, kThreads>(qt.dout, dO + lrow * ld + h * D, ld, nq, tid);
        if constexpr (sizeof(T) == 2) {
          stage_rows_t<D, BQ, kThreads>(qt.qt, Q + lrow * ld + h * D, ld, nq, tid);
          stage_rows_t<D, BQ, kThreads>(qt.doutt, dO + lrow * ld + h * D, ld, nq, tid);
        }
        for (int j = tid; j < BQ; j += kThreads) qt.ts[j] = j < nq ? p.ts[seq0 + q0 + j] : 0;
        __syncthreads();

        float pv[BQ / 32][16], gv[BQ / 32][16];
#pragma unroll
        for (int blk = 0; blk < BQ / 32; ++blk) {
          const f32x16 s = mma_tile_rows<T, D>(qt.q, blk * 32 + r32, kop, g);
          const f32x16 dp = mma_tile_rows<T, D>(qt.dout, blk * 32 + r32, vop, g);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qj = blk * 32 + acc_row(i, g);
            const bool valid = kvalid && qj < nq && kpos <= q0 + qj;
            const int bk = bucket_of(qt.ts[qj] - tsk, p.NB, nb32, tb.e);
            const float x = fmaf(s[i], p.alpha, tb.w[bk]);
            const float sg_ = fast_sigmoid(x);
            float a = x * sg_;
            float gg = p.alpha * dp[i] * (sg_ * (1.0f + x * (1.0f - sg_)));
            if (!valid) {
              a = 0.0f;
              gg = 0.0f;
            } else {
              atomicAdd(&tb.dw[bk], gg);
            }
            pv[blk][i] = a;
            gv[blk][i] = gg;
          }
        }
        if constexpr (sizeof(T) == 2) {
          mma_contract_rows<T, D, BQ>(dvacc, qt.doutt, pv, r32, g);
          mma_contract_rows<T, D, BQ>(dkacc, qt.qt, gv, r32, g);
        } else {
          mma_contract_rows<T, D, BQ>(dvacc, qt.dout, pv, r32, g);
          mma_contract_rows<T, D, BQ>(dkacc, qt.q, gv, r32, g);
        }
      }
    }
    if (kvalid) {
      store_row_from_acc<T, D>(dK + krow * ld + h * D, dkacc, g);
      store_row_from_acc<T, D>(dV + krow * ld + h * D, dvacc, g);
    }
    __syncthreads();
    for (int i = tid; i < p.NB; i += kThreads) {
      const float v = tb.dw[i];
      if (v != 0.0f) atomicAdd(p.dw + (int64_t)h * p.NB + i, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major pass: dQ.  Same item list and lane ownership as the
// forward; Sᵀ = K Qᵀ and dPᵀ = V dOᵀ are recomputed and dQᵀ += Kᵀ Gᵀ.
// ---------------------------------------------------------------------------
template <typename T, int D, int BN> struct alignas(16) KvtTiles {
  T k[BN * Pitch<T, D>::row];
  T v[BN * Pitch<T, D>::row];
  T kt[sizeof(T) == 2 ? D * TPitch<BN>::col : 1];
  int64_t ts[BN];
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_q_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  constexpr int BN = FwdCfg<T, D>::BN;
  __shared__ KvtTiles<T, D, BN> kv;
  __shared__ Tables tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  const int H = p.H;
  const float nb32 = p.NB * (1.0f / 32.0f);
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
    for (int kt = 0; kt < n_kt; ++kt) {
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      __syncthreads();
      const int64_t krow = seq0 + key0;
      stage_rows<T, D, BN, kThreads>(kv.k, K + krow * ld + h * D, ld, nvalid, tid);
      stage_rows<T, D, BN, kThreads>(kv.v, V + krow * ld + h * D, ld, nvalid, tid);
      if constexpr (sizeof(T) == 2) stage_rows_t<D, BN, kThreads>(kv.kt, K + krow * ld + h * D, ld, nvalid, tid);
      for (int j = tid; j < BN; j += kThreads) kv.ts[j] = j < nvalid ? p.ts[krow + j] : 0;
      __syncthreads();

      float gv[BN / 32][16];
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) {
        const f32x16 s = mma_tile_rows<T, D>(kv.k, blk * 32 + r32, qop, g);
        const f32x16 dp = mma_tile_rows<T, D>(kv.v, blk * 32 + r32, dop, g);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = blk * 32 + acc_row(i, g);
          const int bk = bucket_of(tsq - kv.ts[kj], p.NB, nb32, tb.e);
          const float x = fmaf(s[i], p.alpha, tb.w[bk]);
          const float sg_ = fast_sigmoid(x);
          float gg = p.alpha * dp[i] * (sg_ * (1.0f + x * (1.0f - sg_)));
          if (key0 + kj > qpos || !qvalid) gg = 0.0f;
          gv[blk][i] = gg;
        }
      }
      if constexpr (sizeof(T) == 2)
        mma_contract_rows<T, D, BN>(dqacc, kv.kt, gv, r32, g);
      else
        mma_contract_rows<T, D, BN>(dqacc, kv.k, gv, r32, g);
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

int attn_q_tile_rows() { return FwdCfg<float, 128>::BM; }
int attn_k_tile_keys() { return FwdCfg<float, 128>::BN; }
int attn_bwd_key_tile() { return BwdKvCfg<float, 128>::BK; }
int attn_bwd_q_step() { return BwdKvCfg<float, 128>::BQ; }

}  // namespace hstu
