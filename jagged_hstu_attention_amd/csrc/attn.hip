// Jagged HSTU attention kernels for gfx950: forward, dK/dV/d(ts_weights) pass
// and dQ pass.  All three are persistent: every workgroup pops work items
// (tile x head) from a descending-cost list built by the scheduler kernel.
//
// The operation (Scaling Generative Recommendations with Context Parallelism on
// HSTU, §2.1, HSTUAttention equation and timestamp-bias paragraph):
//   x_ij = alpha * (q_i . k_j + w[h, bucket(ts_i - ts_j)]),  alpha = 1/sqrt(d)
//   a_ij = SiLU(x_ij) * [pos_j <= pos_i]
//   O_i  = sum_j a_ij v_j
// Backward: dP = dO Vᵀ, G = alpha * dP * SiLU'(x) * mask, dV = aᵀ dO,
// dK = Gᵀ Q, dQ = G K, dW[h, b] = sum of G over pairs in bucket b.
//
// Arithmetic per score: with y = -log2(e) * x (one fma from the raw dot
// product and a pre-scaled bias table), sigma = 1 / (1 + 2^y) and a' = y sigma
// = -log2(e) SiLU(x).  SiLU'(x) = sigma + x sigma (1 - sigma)
// = sigma - ln2 * a' (1 - sigma).  The constant factors -ln 2 (of a') and
// alpha (of G) are applied once to the accumulated outputs.
//
// Every lane owns one row for the whole item (a query in the forward and dQ
// passes, a key in the dK/dV pass), so the timestamp of its row, its causal
// limit and its bias plan (bias.h) are per-lane scalars.  The other side
// streams through double-buffered, swizzled LDS tiles (swtile.h) filled with
// direct-to-LDS loads one tile ahead; one barrier per tile.  Each tile is
// processed by a branch-free body specialised for its bias mode and for
// whether it needs the causal mask.
#include "attn.h"
#include "bias.h"
#include "swtile.h"

namespace hstu {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int BM = 128;        // query rows per forward / dQ item (32 per wave)
constexpr int BN = 64;         // keys per tile in the forward / dQ loops
constexpr int BK = 128;        // keys per dK/dV item (32 per wave)
constexpr int BQ = 64;         // query rows per step of the dK/dV loop
static_assert(BQ == BN, "the dK/dV step tiles share the key-tile shape");

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

// d(ts_weights) bins are kept in kDwCopies copies (lane l adds to copy
// l % kDwCopies): neighbouring keys usually share a bucket, so lanes of one
// atomic instruction would otherwise collide on one address.  The copies are
// summed at flush time.
template <typename T, int D>
constexpr int kDwCopies = sizeof(T) == 2 ? 32 : 8;  // fp32, d = 128 has no LDS left for more

// MFMA products against LDS tiles, per element type.
template <typename T, int D> struct TileOps;

template <int D> struct TileOps<__bf16, D> {
  LaneOffsets<D> lo;
  __device__ __forceinline__ void init(int lane) { lo.init(lane); }
  __device__ __forceinline__ f32x16 rows(const __bf16* t, int blk, const bf16x8* op) const {
    return tile_mma_rows_o<D>(reinterpret_cast<const char*>(t), lo, blk, op);
  }
  // rows(a, blk, opa) and rows(b, blk, opb) as one stream: the LDS operands
  // of slice kk + 1 are read while the two MFMAs of slice kk run
  __device__ __forceinline__ void rows2(f32x16& ra, f32x16& rb, const __bf16* a, const __bf16* b, int blk,
                                        const bf16x8* opa, const bf16x8* opb) const {
    const char* pa = reinterpret_cast<const char*>(a) + blk * 32 * D * 2;
    const char* pb = reinterpret_cast<const char*>(b) + blk * 32 * D * 2;
    ra = f32x16{};
    rb = f32x16{};
    u32x4 xa = *reinterpret_cast<const u32x4*>(pa + lo.row[0]);
    u32x4 xb = *reinterpret_cast<const u32x4*>(pb + lo.row[0]);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 ya = xa, yb = xb;
      if (kk + 1 < D / 16) {
        ya = *reinterpret_cast<const u32x4*>(pa + lo.row[kk + 1]);
        yb = *reinterpret_cast<const u32x4*>(pb + lo.row[kk + 1]);
      }
      ra = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, xa), opa[kk], ra);
      rb = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, xb), opb[kk], rb);
      __builtin_amdgcn_sched_barrier(0);
      xa = ya;
      xb = yb;
    }
  }
  __device__ __forceinline__ void contract(f32x16* out, const __bf16* t, const float* vals, int blk) const {
    tile_contract_block_o<D>(out, reinterpret_cast<const char*>(t), lo, vals, blk);
  }
};

template <int D> struct TileOps<float, D> {
  int lane;
  __device__ __forceinline__ void init(int l) { lane = l; }
  __device__ __forceinline__ f32x16 rows(const float* t, int blk, const float* op) const {
    return tile_mma_rows<float, D>(t, blk * 32 + (lane & 31), op, lane >> 5);
  }
  __device__ __forceinline__ void contract(f32x16* out, const float* t, const float* vals, int blk) const {
    tile_contract_block<float, D>(out, t, vals, blk, lane);
  }
};

template <typename T, int D> struct alignas(16) KvSmem {
  T k[2][BN * D];
  T v[2][BN * D];
};

template <typename T, int D, int NT = kThreads>
__device__ __forceinline__ void issue_kv(KvSmem<T, D>& sm, int buf, const T* Kh, const T* Vh, int64_t ld, int key0,
                                         int nvalid, int tid, uint32_t lane_off) {
  tile_load_async<T, D, BN, NT>(sm.k[buf], Kh + key0 * ld, ld, nvalid, tid, lane_off);
  tile_load_async<T, D, BN, NT>(sm.v[buf], Vh + key0 * ld, ld, nvalid, tid, lane_off);
}

// The exact-bucket table and edges (once per workgroup) ...
template <int NT = kThreads>
__device__ __forceinline__ void load_bucket_tables(BiasLds& bl, const AttnParams& p, int tid) {
  for (int i = tid; i < kLutSize; i += NT) bl.lut[i] = p.lut[i];
  for (int i = tid; i < p.NB + kPad; i += NT)
    bl.e[i] = i <= p.NB ? (int32_t)min(p.edges[i], 0x7FFFFFFFu) : 0x7FFFFFFF;
}

// ... and the head's scaled bias values (per item).
template <typename T, int NT = kThreads>
__device__ __forceinline__ void load_bias_values(BiasLds& bl, const AttnParams& p, int h, int tid) {
  const T* W = static_cast<const T*>(p.w) + (int64_t)h * p.NB;
  const float s = kNegLog2e * p.alpha;
  for (int i = tid; i < p.NB + kPad; i += NT) bl.c[i] = s * to_f32<T>(W[min(i, p.NB - 1)]);
}

// The item index is read back from LDS; readfirstlane marks it wave-uniform,
// so everything derived from it (item fields, offsets, tile bases) lives in
// scalar registers.
__device__ __forceinline__ int pop_item(int* slot, int* counter, int tid) {
  __syncthreads();
  if (tid == 0) *slot = atomicAdd(counter, 1);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);
}

// d(ts_weights): the dK/dV pass, which ran before the dQ pass on the same
// stream, left the finished sums in the workspace; workgroup 0 of the dQ pass
// copies them to the output.
template <int NT = kThreads>
__device__ __forceinline__ void publish_dw(const AttnParams& p, int tid) {
  if (blockIdx.x == 0 && p.dw)
    for (int i = tid; i < p.H * p.NB; i += NT) p.dw[i] = p.dw_acc[i];
}

// Lane timestamp relative to the item base, and whether every valid lane of
// the wave is within 2^30 of it (then the 32-bit paths apply to tiles that are
// not wide).
struct LaneTs {
  int32_t rel;
  bool fast;
};
__device__ __forceinline__ LaneTs lane_ts(int64_t ts, bool valid, int64_t base) {
  const int64_t d = ts - base;
  const bool ok = !valid || (d > -(1ll << 30) && d < (1ll << 30));
  LaneTs r;
  r.fast = __ballot(!ok) == 0;
  r.rel = valid && ok ? (int32_t)d : 0;
  return r;
}

// y = -log2(e) x, sigma = 1 / (1 + 2^y).
__device__ __forceinline__ float sigmoid_y(float y) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y)); }

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

__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
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
    // the fields derive from wave-uniform values; readfirstlane keeps them in
    // scalar registers (as vector registers they could be spilled, and every
    // scratch reload waits for all outstanding loads, the tile prefetch too)
    r0 = uni64(r0);
    r1 = uni64(r1);
    p0 = __builtin_amdgcn_readfirstlane(p0);
    p1 = __builtin_amdgcn_readfirstlane(p1);
    e0 = __builtin_amdgcn_readfirstlane(e0);
    e1 = __builtin_amdgcn_readfirstlane(e1);
    nseg = __builtin_amdgcn_readfirstlane(nseg);
    start = __builtin_amdgcn_readfirstlane(start);
    si = __builtin_amdgcn_readfirstlane(si);
    q0 = __builtin_amdgcn_readfirstlane(q0);
  }
  __device__ __forceinline__ bool valid() const { return si < nseg; }
  __device__ __forceinline__ int nq() const { return min(BQ, seg_end(si) - q0); }
  __device__ __forceinline__ int64_t lrow() const { return (si == 0 ? r0 : r1) + (q0 - seg_pos(si)); }
  __device__ __forceinline__ void next() {
    q0 += BQ;
    norm();
  }
};

// Scale an accumulator set and store it as one row.
template <typename T, int D>
__device__ __forceinline__ void store_scaled(T* dst, f32x16* acc, float s, int g) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] *= s;
  store_row_from_acc<T, D>(dst, acc, g);
}

}  // namespace

// ---------------------------------------------------------------------------
// Forward.  One item = (query tile of 128 rows, head).  Wave w owns query rows
// 32w..32w+31 of the tile; lane (r32, g) owns query row 32w + r32: the score
// tile is computed transposed, Sᵀ = K Qᵀ, so every accumulator value of a lane
// belongs to its own query, and the output is Oᵀ = Vᵀ Pᵀ with P taken straight
// from the Sᵀ accumulators (V read with transpose reads).
// ---------------------------------------------------------------------------
namespace {

struct FwdLane {
  int32_t tsr;      // own timestamp relative to the item base (32-bit modes)
  int64_t ts64;     // own timestamp
  int lim;          // key rows > lim of the tile are masked (qpos - key0)
  int hlim;         // key rows >= hlim other than lim are candidates, masked (history end - key0)
  int g;
  float beta;       // -log2(e) * alpha
  int nb;
};

// a' = y sigma(y) for the 16 values of one block, y = beta s + cb.  Masked:
// key row r of the block is visible iff r <= lim and (r < hlim or r == lim).
template <bool MASK>
__device__ __forceinline__ void silu_block(float* pv, const f32x16& s, const float* cb, float beta, int lim, int hlim,
                                           int g) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = fmaf(s[i], beta, cb[i]);
    const float a = y * sigmoid_y(y);
    const int r = acc_row(i, g);
    pv[i] = (MASK && (r > lim || (r >= hlim && r != lim))) ? 0.0f : a;
  }
}

// One 64-key tile: per 32-key block, the score MFMAs, the block's bias (their
// latency overlaps), SiLU and the P V MFMAs; `mid` runs between the blocks.
template <typename T, int D, bool MASK, typename Mid>
__device__ __forceinline__ void fwd_tile(f32x16* oacc, const T* kt, const T* vt, const TsTile<BN>& ts,
                                         const TileOps<T, D>& ops, const typename Mma<T>::operand* qop, int mode,
                                         const Plan& pl, const FwdLane& ln, const BiasLds& bl, Mid&& mid) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f32x16 s;
    bf16x8 tv[D / 16];
    if constexpr (sizeof(T) == 2) {
      // all K operands of the block, then its MFMAs; the V operands of the
      // P V product are read while the bias and SiLU are computed
      bf16x8 ka[D / 16];
      rows_load<D>(ka, reinterpret_cast<const char*>(kt), ops.lo, blk);
      __builtin_amdgcn_sched_barrier(0);
      s = rows_mma<D>(ka, qop);
      tr_load<D>(tv, reinterpret_cast<const char*>(vt), ops.lo, blk);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      s = ops.rows(kt, blk, qop);
    }
    float cb[16];
    block_bias_mode<+1, BN, false, MASK>(cb, nullptr, mode, pl, ln.tsr, ln.ts64, ts, blk, ln.g, bl, ln.nb);
    if (blk == 1) mid();
    float pv[16];
    silu_block<MASK>(pv, s, cb, ln.beta, ln.lim - 32 * blk, ln.hlim - 32 * blk, ln.g);
    if constexpr (sizeof(T) == 2)
      tr_mma<D>(oacc, tv, pv);
    else
      ops.contract(oacc, vt, pv, blk);
  }
}

}  // namespace

// bf16 with d <= 64 fits three workgroups per compute unit (the register cap
// of 168 costs a few spills, the third wave per SIMD hides more latency)
template <typename T, int D> constexpr int kFwdBlocks = sizeof(T) == 2 && D <= 64 ? 3 : 2;

template <typename T, int D>
__global__ __launch_bounds__(kThreads, (kFwdBlocks<T, D>)) void fwd_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  __shared__ KvSmem<T, D> sm;
  __shared__ TsTile<BN> tsm[2];
  __shared__ BiasLds bl;
  __shared__ int item_slot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  TileOps<T, D> ops;
  ops.init(lane);
  const int H = p.H, NB = p.NB;
  const int64_t ld = (int64_t)H * D;
  const uint32_t lane_off = tile_lane_offset<T, D, kThreads>(tid, ld);
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  T* O = static_cast<T*>(p.out);
  load_bucket_tables(bl, p, tid);
  const int n_work = p.ctr[kCtrQTiles] * H;

  for (;;) {
    const int w = pop_item(&item_slot, p.ctr + kCtrQNext, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.qitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int64_t base = p.ts[seq0];
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
    load_bias_values<T>(bl, p, h, tid);
    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};

    const int kv_len = it.pos0 + it.n;
    const int wave_qmin = it.pos0 + wave * 32;
    // Key tiles visited: the causal prefix [0, ht) over the history rows,
    // then, past the history, only the tiles [d0, last] that hold the item's
    // own rows (a candidate sees no other candidate).  Without candidates
    // hist is the sequence length and the walk is 0 .. last.
    int hist = kv_len;
    if (p.num_targets) {  // candidates clamped to [0, L], as the scheduler does
      const int L = (int)(p.offsets[it.b + 1] - seq0);
      hist = L - (int)min(max(p.num_targets[it.b], (int64_t)0), (int64_t)L);
    }
    const int ht = (min(kv_len, hist) + BN - 1) / BN, last = (kv_len - 1) / BN;
    const int d0 = kv_len <= hist ? last + 1 : max(max(it.pos0, hist) / BN, ht);
    const T* Kh = K + seq0 * ld + h * D;
    const T* Vh = V + seq0 * ld + h * D;
    const LaneTs lt = lane_ts(tsq, qvalid, base);
    FwdLane ln;
    ln.g = g;
    ln.beta = kNegLog2e * p.alpha;
    ln.nb = NB;
    ln.ts64 = tsq;
    ln.tsr = lt.rel;
    // key tile at position pos of the walk; the item covers positions
    // [it.w0, it.w1) (the whole walk unless the tile is split)
    const auto walk = [&](int pos) { return pos < ht ? pos : d0 + (pos - ht); };
    // wave 0 reads the timestamps of a tile one step before it stages them
    // (half-way through the tile before), so staging never waits for the
    // tile loads in flight
    const auto tile_ts = [&](int pos) {
      const int k0 = walk(pos) * BN;
      return p.ts[seq0 + k0 + min(lane, min(BN, kv_len - k0) - 1)];
    };
    int64_t tsv = 0;
    int kt = walk(it.w0);
    {
      const int nv0 = min(BN, kv_len - kt * BN);
      issue_kv<T, D>(sm, 0, Kh, Vh, ld, kt * BN, nv0, tid, lane_off);
      if (wave == 0) {
        const int64_t t0 = tile_ts(it.w0);
        if (it.w0 + 1 < it.w1) tsv = tile_ts(it.w0 + 1);
        ts_tile_fill<BN>(tsm[0], t0, nv0, lane, base);
      }
    }
    wait_loads();
    __syncthreads();
    for (int pos = it.w0; pos < it.w1; ++pos) {
      const int cur = (pos - it.w0) & 1;
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      const int nkt = walk(pos + 1);
      const bool more = pos + 1 < it.w1;
      const int nk0 = nkt * BN, nnv = more ? min(BN, kv_len - nk0) : 0;
      int64_t tsn = 0;
      if (more) {
        if (wave == 0 && pos + 2 < it.w1) tsn = tile_ts(pos + 2);
        __builtin_amdgcn_sched_barrier(0);
        issue_kv<T, D>(sm, cur ^ 1, Kh, Vh, ld, nk0, nnv, tid, lane_off);
      }
      const auto stage = [&] {
        if (more && wave == 0) ts_tile_fill<BN>(tsm[cur ^ 1], tsv, nnv, lane, base);
      };
      const TsTile<BN>& ts = tsm[cur];
      const int4 hdr = ts.hdr;
      const bool fast = lt.fast && hdr.z == 0;
      ln.lim = qpos - key0;
      ln.hlim = hist - key0;
      if (key0 + BN - 1 > wave_qmin || nvalid < BN || !fast || key0 + BN > hist) {
        fwd_tile<T, D, true>(oacc, sm.k[cur], sm.v[cur], ts, ops, qop, fast ? kModeLut : kModeWide, Plan{}, ln, bl,
                             stage);
      } else {
        const Plan pl = make_plan<+1>(ln.tsr, qvalid, hdr.x, hdr.y, bl);
        fwd_tile<T, D, false>(oacc, sm.k[cur], sm.v[cur], ts, ops, qop, wave_mode(pl.n), pl, ln, bl, stage);
      }
      wait_loads();
      __syncthreads();
      kt = nkt;
      tsv = tsn;
    }
    if (qvalid) {
      if (it.slot < 0)
        store_scaled<T, D>(O + qrow * ld + h * D, oacc, kNegLn2, g);
      else
        store_row_from_acc<float, D>(p.parts + ((int64_t)it.slot * H + h) * kSplitRows * D + (int64_t)qi * D, oacc, g);
    }
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
namespace {

struct KvLane {
  int32_t tsr;
  int64_t ts64;
  int lo_row;   // query rows r of the step are visible iff lo_row <= r < hi_row
  int hi_row;
  int g;
  float beta;
  int nb;
  bool valid;
};

// d(ts_weights) sums of a plan-mode step: s0 = all G, s_k = G passing edge k.
struct DwSums {
  float s0, s1, s2, s3;
};

template <typename T, int D, bool MASK>
__device__ __forceinline__ void kv_tile(f32x16* dkacc, f32x16* dvacc, DwSums& dws, float* dwl, const T* qt,
                                        const T* dt, const TsTile<BQ>& ts, const TileOps<T, D>& ops,
                                        const typename Mma<T>::operand* kop, const typename Mma<T>::operand* vop,
                                        int mode, const Plan& pl, const KvLane& ln, const BiasLds& bl) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const f32x16 s = ops.rows(qt, blk, kop);
    const f32x16 dp = ops.rows(dt, blk, vop);
    float cb[16];
    int key[16];
    block_bias_mode<-1, BQ, true, MASK>(cb, key, mode, pl, ln.tsr, ln.ts64, ts, blk, ln.g, bl, ln.nb);
    float pv[16], gv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float y = fmaf(s[i], ln.beta, cb[i]);
      const float sg = sigmoid_y(y);
      const float a = y * sg;
      const float u = fmaf(-a, sg, a);  // a' (1 - sigma)
      const float gg = dp[i] * fmaf(u, kNegLn2, sg);
      bool vis = true;
      if constexpr (MASK) {
        const int r = acc_row(i, ln.g) + blk * 32;
        vis = r >= ln.lo_row && r < ln.hi_row;
      }
      pv[i] = vis ? a : 0.0f;
      gv[i] = vis ? gg : 0.0f;
    }
    ops.contract(dvacc, dt, pv, blk);
    ops.contract(dkacc, qt, gv, blk);
    // d(ts_weights): exact modes add per element (masked-out elements skip
    // the atomic), plan modes keep sums
    if (MASK || mode >= kModeLut) {
      if (ln.valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) atomicAdd(&dwl[key[i]], gv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) dws.s0 += gv[i];
      if (mode != kModeConst) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dws.s1 += key[i] >= 1 ? gv[i] : 0.0f;
        if (mode == kModeThr3) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            dws.s2 += key[i] >= 2 ? gv[i] : 0.0f;
            dws.s3 += key[i] >= 3 ? gv[i] : 0.0f;
          }
        }
      }
    }
  }
}

// Plan-mode step specialised for its mode (constant bias, one or up to three
// thresholds): the whole step is one basic block in which the compiler can
// interleave the MFMAs with the elementwise work; the d(ts_weights) sums are
// kept for the thresholds the mode has.
template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_tile_plan(f32x16* dkacc, f32x16* dvacc, DwSums& dws, const T* qt, const T* dt,
                                             const TsTile<BQ>& ts, const TileOps<T, D>& ops,
                                             const typename Mma<T>::operand* kop,
                                             const typename Mma<T>::operand* vop, const float c0, const float c1,
                                             const float c2, const float c3, const int32_t t1, const int32_t t2,
                                             const int32_t t3, const int flip, const float beta) {
  const int32_t* varr = ts.un[flip ? 1 : 0];
  const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const f32x16 s = ops.rows(qt, blk, kop);
    const f32x16 dp = ops.rows(dt, blk, vop);
    int32_t v[16];
    if constexpr (MODE != kModeConst) block_rows_i32(v, varr, blk, g);
    float pv[16], gv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float c = c0;
      bool p1 = false, p2 = false, p3 = false;
      if constexpr (MODE != kModeConst) {
        p1 = v[i] <= t1;
        c = p1 ? c1 : c;
      }
      if constexpr (MODE == kModeThr3) {
        p2 = v[i] <= t2;
        p3 = v[i] <= t3;
        c = p2 ? c2 : c;
        c = p3 ? c3 : c;
      }
      const float y = fmaf(s[i], beta, c);
      const float sg = sigmoid_y(y);
      const float a = y * sg;
      const float u = fmaf(-a, sg, a);  // a' (1 - sigma)
      const float gg = dp[i] * fmaf(u, kNegLn2, sg);
      pv[i] = a;
      gv[i] = gg;
      dws.s0 += gg;
      if constexpr (MODE != kModeConst) dws.s1 += p1 ? gg : 0.0f;
      if constexpr (MODE == kModeThr3) {
        dws.s2 += p2 ? gg : 0.0f;
        dws.s3 += p3 ? gg : 0.0f;
      }
    }
    ops.contract(dvacc, dt, pv, blk);
    ops.contract(dkacc, qt, gv, blk);
  }
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_kv_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  __shared__ KvSmem<T, D> sm;  // k: query rows, v: dO rows
  __shared__ TsTile<BN> tsm[2];
  __shared__ BiasLds bl;
  constexpr int kCopies = kDwCopies<T, D>;
  __shared__ float dwbins[kCopies][kMaxBuckets + 1];
  __shared__ int item_slot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  TileOps<T, D> ops;
  ops.init(lane);
  const int H = p.H, NB = p.NB;
  const int64_t ld = (int64_t)H * D;
  const uint32_t lane_off = tile_lane_offset<T, D, kThreads>(tid, ld);
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* dO = static_cast<const T*>(p.dout);
  T* dK = static_cast<T*>(p.dk);
  T* dV = static_cast<T*>(p.dv);
  load_bucket_tables(bl, p, tid);
  const int n_work = p.ctr[kCtrKTiles] * H;
  float* dwl = dwbins[lane % kCopies];

  for (;;) {
    const int w = pop_item(&item_slot, p.ctr + kCtrKNext, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.kitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int64_t base = p.ts[seq0];
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
    load_bias_values<T>(bl, p, h, tid);
    for (int i = tid; i < kCopies * (kMaxBuckets + 1); i += kThreads) (&dwbins[0][0])[i] = 0.0f;
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      dkacc[i] = f32x16{};
      dvacc[i] = f32x16{};
    }
    const int wave_kmax = it.pos0 + wave * 32 + 31;
    const LaneTs lt = lane_ts(tsk, kvalid, base);
    KvLane ln;
    ln.g = g;
    ln.beta = kNegLog2e * p.alpha;
    ln.nb = NB;
    ln.ts64 = tsk;
    ln.tsr = lt.rel;
    ln.valid = kvalid;

    int64_t tsv = 0;
    StepIter si;
    si.init(p, it.b, it.pos0);
    int cur = 0;
    if (si.valid()) {
      issue_kv<T, D>(sm, 0, Q + h * D, dO + h * D, ld, (int)si.lrow(), si.nq(), tid, lane_off);
      if (wave == 0) tsv = p.ts[seq0 + si.q0 + min(lane, si.nq() - 1)];
      if (wave == 0) ts_tile_fill<BQ>(tsm[0], tsv, si.nq(), lane, base);
    }
    wait_loads();
    __syncthreads();
    while (si.valid()) {
      const int q0 = si.q0;
      const int nq = si.nq();
      StepIter nx = si;
      nx.next();
      if (nx.valid()) {
        issue_kv<T, D>(sm, cur ^ 1, Q + h * D, dO + h * D, ld, (int)nx.lrow(), nx.nq(), tid, lane_off);
        if (wave == 0) tsv = p.ts[seq0 + nx.q0 + min(lane, nx.nq() - 1)];
      }
      const TsTile<BQ>& ts = tsm[cur];
      const int4 hdr = ts.hdr;
      const bool fast = lt.fast && hdr.z == 0;
      ln.lo_row = kpos - q0;
      ln.hi_row = nq;
      DwSums dws{0.0f, 0.0f, 0.0f, 0.0f};
      if (q0 < wave_kmax || nq < BQ || !fast) {
        kv_tile<T, D, true>(dkacc, dvacc, dws, dwl, sm.k[cur], sm.v[cur], ts, ops, kop, vop,
                            fast ? kModeLut : kModeWide, Plan{}, ln, bl);
      } else {
        const Plan pl = make_plan<-1>(ln.tsr, kvalid, hdr.x, hdr.y, bl);
        const int mode = wave_mode(pl.n);
#define HSTU_KV_PLAN(M)                                                                                        \
  kv_tile_plan<T, D, M>(dkacc, dvacc, dws, sm.k[cur], sm.v[cur], ts, ops, kop, vop, pl.c0, pl.c1, pl.c2, pl.c3, \
                        pl.t1, pl.t2, pl.t3, pl.flip, ln.beta)
        if (mode == kModeConst)
          HSTU_KV_PLAN(kModeConst);
        else if (mode == kModeThr1)
          HSTU_KV_PLAN(kModeThr1);
        else if (mode == kModeThr3)
          HSTU_KV_PLAN(kModeThr3);
        else
          kv_tile<T, D, false>(dkacc, dvacc, dws, dwl, sm.k[cur], sm.v[cur], ts, ops, kop, vop, mode, pl, ln, bl);
#undef HSTU_KV_PLAN
        if (mode < kModeLut && kvalid) {
          // bins b_lo + k from the nested sums
          const int b0 = pl.blo;
          if (dws.s0 != dws.s1) atomicAdd(&dwl[b0], dws.s0 - dws.s1);
          if (dws.s1 != dws.s2) atomicAdd(&dwl[b0 + 1], dws.s1 - dws.s2);
          if (dws.s2 != dws.s3) atomicAdd(&dwl[b0 + 2], dws.s2 - dws.s3);
          if (dws.s3 != 0.0f) atomicAdd(&dwl[b0 + 3], dws.s3);
        }
      }
      if (nx.valid() && wave == 0) ts_tile_fill<BQ>(tsm[cur ^ 1], tsv, nx.nq(), lane, base);
      wait_loads();
      __syncthreads();
      si = nx;
      cur ^= 1;
    }
    if (kvalid) {
      store_scaled<T, D>(dK + krow * ld + h * D, dkacc, p.alpha, g);
      store_scaled<T, D>(dV + krow * ld + h * D, dvacc, kNegLn2, g);
    }
    for (int i = tid; i < NB; i += kThreads) {
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) v += dwbins[c][i];
      if (v != 0.0f) atomicAdd(p.dw_acc + (int64_t)h * NB + i, p.alpha * v);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, key-major pass for bf16 with d in {64, 128}: items of 128 keys,
// eight waves per workgroup, one workgroup per CU (two waves per SIMD).
// Waves w and w ^ 4 share keys 32 (w % 4) .. + 31.  In every step of 64 query
// rows, wave w computes S and dP only for the 32-row block hf = w / 4, and the
// pair swaps the resulting P and G through LDS; each wave then accumulates dV
// and dK over both blocks for its half hf of the head dimension.  A wave so
// holds half the accumulators a full-width wave would and fits in 256
// registers.  The query/dO tiles are double-buffered: the next step's tiles
// load during the whole current step.  A wave whose block lies entirely before
// its first key (the diagonal steps) skips its products: its P and G are zero.
// ---------------------------------------------------------------------------
namespace {

// Per-lane LDS byte offsets of the tile reads of this kernel, compressed: the
// swizzle puts the row read of contraction slice kk at row0 ^ (kk << 5), the
// transpose read of d block j at tr0[h] ^ (j << 6), and rows 16 apart at a
// constant distance (D = 64 and 128).  The kernel passes the three registers
// through an empty asm statement at every step, so that the compiler derives
// the offsets there instead of keeping each of them in a register of its own
// for the whole kernel.
struct HalfOffsets {
  int row0;
  int tr0[2];
  template <int D> __device__ __forceinline__ void init(int lane) {
    using S = SwTile<__bf16, D>;
    const int r32 = lane & 31, g = lane >> 5, m = lane & 15, q = lane >> 4;
    row0 = 2 * S::off(r32, 8 * g);
    const int rb = 4 * g + (m >> 2), cb = 16 * (q & 1) + 4 * (m & 3);
    tr0[0] = 2 * S::off(rb, cb);
    tr0[1] = 2 * S::off(rb + 8, cb);
  }
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(row0), "+v"(tr0[0]), "+v"(tr0[1])); }
};

// out[j] += Xᵀ (d block j of the half) B over the 32 rows of block blk of a
// bf16 tile; B is the pair of packed bf16x8 operands of the block.
template <int D>
__device__ __forceinline__ void contract_half(f32x16* out, const char* __restrict__ base, const HalfOffsets& o, int hf,
                                              const u32x4* b, int blk) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int jj = hf * (D / 64) + j;  // d block of the head
      const char* p0 = base + (o.tr0[0] ^ (jj << 6)) + (blk * 32 + 16 * u) * D * 2;
      const char* p1 = base + (o.tr0[1] ^ (jj << 6)) + (blk * 32 + 16 * u) * D * 2;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const short __attribute__((ext_vector_type(8))) a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      out[j] = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b[u]), out[j]);
    }
}

// S = Q Kᵀ (K operands in registers) and dP = dO Vᵀ (V rows from LDS) for
// block blk of the query/dO tiles, the LDS operands of slice kk + 1 read while
// the MFMAs of slice kk run.
template <int D>
__device__ __forceinline__ void sdp_products(f32x16& s, f32x16& dp, const char* __restrict__ qb,
                                             const char* __restrict__ db, const char* __restrict__ vb,
                                             const HalfOffsets& o, int blk, int vblk, const bf16x8* kop) {
  s = f32x16{};
  dp = f32x16{};
  const int qo = blk * 32 * D * 2, vo = vblk * 32 * D * 2;
  u32x4 qa = *reinterpret_cast<const u32x4*>(qb + o.row0 + qo);
  u32x4 da = *reinterpret_cast<const u32x4*>(db + o.row0 + qo);
  u32x4 va = *reinterpret_cast<const u32x4*>(vb + o.row0 + vo);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 qn = qa, dn = da, vn = va;
    if (kk + 1 < D / 16) {
      const int r = o.row0 ^ ((kk + 1) << 5);
      qn = *reinterpret_cast<const u32x4*>(qb + r + qo);
      dn = *reinterpret_cast<const u32x4*>(db + r + qo);
      vn = *reinterpret_cast<const u32x4*>(vb + r + vo);
    }
    s = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, qa), kop[kk], s);
    dp = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, da), __builtin_bit_cast(bf16x8, va), dp);
    __builtin_amdgcn_sched_barrier(0);
    qa = qn;
    da = dn;
    va = vn;
  }
}

__device__ __forceinline__ void pack16(u32x4* dst, const float* v) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
    dst[u] = u32x4{pack_bf16x2(v[8 * u], v[8 * u + 1]), pack_bf16x2(v[8 * u + 2], v[8 * u + 3]),
                   pack_bf16x2(v[8 * u + 4], v[8 * u + 5]), pack_bf16x2(v[8 * u + 6], v[8 * u + 7])};
}

// Elementwise part of an unmasked step under a plan mode (kModeConst, Thr1,
// Thr3): each element's bias by compares of the other row's timestamp offset
// (rows[], this lane's four-row runs) with the lane's thresholds, SiLU and its
// gradient, P and G packed to bf16, and the d(ts_weights) contributions summed
// per passed edge into dw4 (bins b_lo .. b_lo + 3; the caller adds them to the
// LDS bins).  An edge the tile does not cross is never passed, so its sum is
// zero.
template <int MODE>
__device__ __forceinline__ void pair_plan(u32x4* own_p, u32x4* own_g, float* dw4, const f32x16& s, const f32x16& dp,
                                          const int32_t* __restrict__ rows, float beta, float c0, float c1, float c2,
                                          float c3, int32_t t1, int32_t t2, int32_t t3) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  float pa[16], pg[16];
  // Runs of four values, each computed stage by stage (the four bias
  // selections, then the four fmas, the four exponentials, ...) with the
  // scheduler held to that order: four independent chains hide the latency
  // of the transcendental steps, which one chain at a time would expose.
  int4 rv[4] = {};  // the other rows' timestamp offsets, all read up front
  if constexpr (MODE != kModeConst)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) rv[q4] = *reinterpret_cast<const int4*>(rows + q4 * 8);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int32_t vv[4] = {rv[q4].x, rv[q4].y, rv[q4].z, rv[q4].w};
    float c[4], y[4], t[4], a[4], h[4];
    bool p1[4] = {false, false, false, false}, p2[4] = {false, false, false, false},
         p3[4] = {false, false, false, false};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = c0;
      if constexpr (MODE != kModeConst) {
        p1[e] = vv[e] <= t1;
        c[e] = p1[e] ? c1 : c[e];
      }
      if constexpr (MODE == kModeThr3) {
        p2[e] = vv[e] <= t2;
        p3[e] = vv[e] <= t3;
        c[e] = p2[e] ? c2 : c[e];
        c[e] = p3[e] ? c3 : c[e];
      }
      y[e] = fmaf(s[4 * q4 + e], beta, c[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_exp2f(y[e]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_rcpf(1.0f + t[e]);  // sigma
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = y[e] * t[e];
      h[e] = fmaf(fmaf(-a[e], t[e], a[e]), kNegLn2, t[e]);  // a' (1 - sigma) (-ln 2) + sigma
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q4 + e;
      pa[i] = a[e];
      pg[i] = dp[i] * h[e];
      s0 += pg[i];
      if constexpr (MODE != kModeConst) s1 += p1[e] ? pg[i] : 0.0f;
      if constexpr (MODE == kModeThr3) {
        s2 += p2[e] ? pg[i] : 0.0f;
        s3 += p3[e] ? pg[i] : 0.0f;
      }
    }
  }
  pack16(own_p, pa);
  pack16(own_g, pg);
  // the contributions to bins b_lo .. b_lo + 3 (an edge the mode does not
  // test contributes nothing)
  dw4[0] = s0 - s1;
  dw4[1] = s1 - s2;
  dw4[2] = s2 - s3;
  dw4[3] = s3;
}

// Elementwise part with the exact bucket per element (32-bit offsets from the
// table, or WIDE: 64-bit timestamps), the causal / row-count mask when MASKED
// (row r of the block is visible iff lo_row <= r < hi_row), and the
// d(ts_weights) contributions summed per run of equal buckets.  A key lane
// past the item's end has dp = 0 (its V operand is zero), so its G and
// contributions vanish.
template <bool WIDE, bool MASKED>
__device__ __forceinline__ void pair_exact(u32x4* own_p, u32x4* own_g, float* dwl, const f32x16& s, const f32x16& dp,
                                           const TsTile<BQ>& ts, int blk, int g, float beta, int32_t tsr,
                                           int64_t tsr64, const BiasLds& bl, int nb, int lo_row, int hi_row) {
  float pa[16], pg[16];
  int cur = 0;        // bucket of the running d(ts_weights) sum
  float run = 0.0f;   // the running sum
  // row r0 + e = 8 q4 + e + 4g is visible iff 8 q4 + e lies in [lo_g, hi_g)
  // (the compile-time part compared with two lane values)
  const int lo_g = lo_row - 4 * g, hi_g = hi_row - 4 * g;
  // Runs of four values, stage by stage (as in pair_plan): the four table
  // lookups of the buckets are in flight together, then the four bias
  // values, then the four SiLU chains.
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int r0 = q4 * 8 + 4 * g;
    uint32_t m[4];
    bool far[4] = {false, false, false, false};  // |delta| >= 2^32: the last bucket
    if constexpr (WIDE) {
      const longlong2* t = reinterpret_cast<const longlong2*>(ts.t64 + blk * 32 + r0);
      const longlong2 a0 = t[0], a1 = t[1];
      const int64_t w64[4] = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t d = w64[e] - tsr64;
        const uint64_t am = d < 0 ? (uint64_t)(-d) : (uint64_t)d;
        far[e] = (am >> 32) != 0;
        m[e] = (uint32_t)am;
      }
    } else {
      const int4 v4 = *reinterpret_cast<const int4*>(ts.un[0] + blk * 32 + r0);
      const int32_t vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t d = vv[e] - tsr;
        m[e] = (uint32_t)(d < 0 ? -d : d);
      }
    }
    // exact bucket: table entry {E, b} of the leading-zero count and the
    // five bits after the leading one; bucket = b + [m >= E] (buckets of 0
    // and 1 agree)
    u32x2 L[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[e] = m[e] > 1u ? m[e] : 1u;
      const int z = __builtin_clz(m[e]);
      L[e] = bl.lut[(z << 5) | (int)(((m[e] << z) >> 26) & 31u)];
    }
    __builtin_amdgcn_sched_barrier(0);
    int b[4];
    float c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = far[e] ? nb - 1 : (int)L[e].y + (m[e] >= L[e].x ? 1 : 0);
      c[e] = bl.c[b[e]];
    }
    __builtin_amdgcn_sched_barrier(0);
    float y[4], t[4], a[4], h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fmaf(s[4 * q4 + e], beta, c[e]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_exp2f(y[e]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = __builtin_amdgcn_rcpf(1.0f + t[e]);  // sigma
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = y[e] * t[e];
      h[e] = fmaf(fmaf(-a[e], t[e], a[e]), kNegLn2, t[e]);  // a' (1 - sigma) (-ln 2) + sigma
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * q4 + e;
      float av = a[e], gg = dp[i] * h[e];
      int bb = b[e];
      if constexpr (MASKED) {
        const bool vis = q4 * 8 + e >= lo_g && q4 * 8 + e < hi_g;
        av = vis ? av : 0.0f;
        gg = vis ? gg : 0.0f;
        if (i > 0) bb = vis ? bb : cur;  // a masked element never ends a run
      }
      pa[i] = av;
      pg[i] = gg;
      // d(ts_weights): a lane's rows come in order and their bucket changes
      // rarely, so each lane keeps a running sum per bucket and adds it to
      // the bins when the bucket changes (one atomic per element would make
      // the lanes that share a bucket collide on one address)
      if (i == 0) {
        cur = bb;
        run = gg;
      } else {
        if (bb != cur) {
          atomicAdd(&dwl[cur], run);
          cur = bb;
          run = 0.0f;
        }
        run += gg;
      }
    }
  }
  atomicAdd(&dwl[cur], run);
  pack16(own_p, pa);
  pack16(own_g, pg);
}

constexpr int kHalfThreads = 512;
constexpr int kHalfKeys = 128;
constexpr int kHalfDwCopies = 4;
static_assert(kHalfDwCopies >= 4, "the row-summed bin updates use one copy per 16-lane row");

// Workgroup barrier for LDS data only: it waits for this wave's LDS accesses
// and not for its global memory operations (a __syncthreads waits for all of
// them, the stored score gradients among them).  A wave whose direct-to-LDS
// loads must be visible waits for them itself first.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D> struct alignas(16) HalfSmem {
  __bf16 q[2][BQ * D];  // this step's and the next step's tiles
  __bf16 d[2][BQ * D];
  __bf16 v[kHalfKeys * D];  // the item's V rows
  TsTile<BQ> ts[2];
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kHalfThreads, 1) void bwd_kv_half_kernel(const AttnParams p) {
  using M = Mma<__bf16>;
  using T = __bf16;
  constexpr int NT = kHalfThreads;
  constexpr int KB = D / 64;
  __shared__ HalfSmem<D> sm;
  __shared__ BiasLds bl;
  __shared__ float dwbins[kHalfDwCopies][kMaxBuckets + kPad];  // plan sums touch up to b_lo + 3
  // per wave: P (2 operands) and G (2 operands), lane-contiguous; each slot
  // padded by 8 entries so that the stored-G gathering reads (below) hit
  // distinct LDS banks
  __shared__ u32x4 xch[8][4][64 + 8];
  __shared__ int item_slot;
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, hf = wave >> 2;
  HalfOffsets ofs;
  ofs.init<D>(lane);
  const int H = p.H, NB = p.NB;
  const int64_t ld = (int64_t)H * D;
  // waves 4-7 load the query/dO tiles (their LDS bin updates are deferred past
  // the load wait, see below); waves 0-3 never have a tile load in flight, so
  // wave 0's timestamp staging waits only for its own timestamp load
  constexpr int NL = NT / 2;
  const bool loader = wave >= 4;
  const uint32_t lane_off = tile_lane_offset<T, D, NL>(tid & (NL - 1), ld);
  const uint32_t lane_off_all = tile_lane_offset<T, D, NT>(tid, ld);
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* dO = static_cast<const T*>(p.dout);
  T* dK = static_cast<T*>(p.dk);
  T* dV = static_cast<T*>(p.dv);
  load_bucket_tables<NT>(bl, p, tid);
  const int n_work = p.ctr[kCtrKTiles] * H;
  float* dwl = dwbins[lane % kHalfDwCopies];
  const float beta = kNegLog2e * p.alpha;
  const bool g_on = p.g && p.ctr[kCtrGMode];  // stored score gradient written by this pass

  for (;;) {
    const int w = pop_item(&item_slot, p.ctr + kCtrKNext, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.kitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int64_t base = p.ts[seq0];
    const int kj = kg * 32 + r32;
    const bool kvalid = kj < it.n;
    const bool partial_keys = 32 * kg + 32 > it.n;  // some key lane of the wave lies past the item's end
    const int kpos = it.pos0 + kj;
    const int64_t krow = (int64_t)it.row0 + kj;
    const int64_t tsk = kvalid ? p.ts[krow] : 0;
    // K operands in registers; the V rows are read from LDS in every step
    bf16x8 kop[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      kop[kk] = bf16x8{};
      if (kvalid) kop[kk] = M::load(K + krow * ld + h * D + kk * 16 + g * 8);
    }
    load_bias_values<T, NT>(bl, p, h, tid);
    for (int i = tid; i < kHalfDwCopies * (kMaxBuckets + kPad); i += NT) (&dwbins[0][0])[i] = 0.0f;
    f32x16 dkacc[KB], dvacc[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      dkacc[i] = f32x16{};
      dvacc[i] = f32x16{};
    }
    const int wave_kmax = it.pos0 + kg * 32 + 31;
    const LaneTs lt = lane_ts(tsk, kvalid, base);
    const T* Qh = Q + h * D;
    const T* dOh = dO + h * D;
    // stored G: this item's blocks start at gbase (query tile 0); the wave's
    // key tile and first row within it
    int64_t gbase = 0;
    if (g_on) {
      const int64_t nt = (p.offsets[it.b + 1] - seq0 + kGRows - 1) / kGRows;
      gbase = p.gblk_off[it.b] + h * nt * (nt + 1);
    }
    const int gkt = (it.pos0 + 32 * kg) / kGKeys, gk0 = (32 * kg) % kGKeys;

    StepIter si;
    si.init(p, it.b, it.pos0);
    int64_t tsv = 0;
    tile_load_async<T, D, kHalfKeys, NT>(sm.v, V + (int64_t)it.row0 * ld + h * D, ld, it.n, tid, lane_off_all);
    if (si.valid()) {
      tile_load_async<T, D, BQ, NT>(sm.q[0], Qh + si.lrow() * ld, ld, si.nq(), tid, lane_off_all);
      tile_load_async<T, D, BQ, NT>(sm.d[0], dOh + si.lrow() * ld, ld, si.nq(), tid, lane_off_all);
      if (wave == 0) tsv = p.ts[seq0 + si.q0 + min(lane, si.nq() - 1)];
    }
    wait_loads();
    if (wave == 0 && si.valid()) ts_tile_fill<BQ>(sm.ts[0], tsv, si.nq(), lane, base);
    __syncthreads();
    const char* vb = reinterpret_cast<const char*>(sm.v);
    const int key_lo = it.pos0 + kg * 32;  // first key of this wave
    int cur = 0;
    while (si.valid()) {
      ofs.opaque();
      const int q0 = si.q0;
      const int nq = si.nq();
      StepIter nx = si;
      nx.next();
      if (nx.valid()) {
        // the next step's timestamps, then its tiles into the other buffers;
        // the timestamps are staged after the elementwise part (waiting for
        // them there leaves the tile loads in flight)
        if (wave == 0) tsv = p.ts[seq0 + nx.q0 + min(lane, nx.nq() - 1)];
        if (loader) {
          tile_load_async<T, D, BQ, NL>(sm.q[cur ^ 1], Qh + nx.lrow() * ld, ld, nx.nq(), tid - NL, lane_off);
          tile_load_async<T, D, BQ, NL>(sm.d[cur ^ 1], dOh + nx.lrow() * ld, ld, nx.nq(), tid - NL, lane_off);
        }
      }
      const char* qb = reinterpret_cast<const char*>(sm.q[cur]);
      const char* db = reinterpret_cast<const char*>(sm.d[cur]);
      const TsTile<BQ>& ts = sm.ts[cur];
      const int4 hdr = ts.hdr;
      const bool fast = lt.fast && hdr.z == 0;
      // rows r of this wave's block are visible iff lo_row <= r < hi_row
      const int lo_row = kpos - q0 - 32 * hf, hi_row = nq - 32 * hf;
      const bool masked = q0 + 32 * hf < wave_kmax || nq < BQ || !fast;
      // a block whose rows all precede the wave's keys (or lie past the step)
      // contributes nothing; the partner's block likewise
      const bool live = q0 + 32 * hf + 31 >= key_lo && 32 * hf < nq;
      const bool par_live = q0 + 32 * (hf ^ 1) + 31 >= key_lo && 32 * (hf ^ 1) < nq;

      u32x4 own_p[2] = {}, own_g[2] = {};
      float dw4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // plan steps: bins blo .. blo + 3, added after the load wait
      int blo = 0;
      if (live) {
        f32x16 s, dp;
        sdp_products<D>(s, dp, qb, db, vb, ofs, hf, kg, kop);
        // rows of the V tile past the item's end repeat its last row: a key
        // lane past the end must have dP = 0 (so G and its d(ts_weights)
        // contributions vanish).  Only a wave whose keys run past the end of
        // the item has such lanes (a wave-uniform test).
        if (partial_keys && !kvalid) dp = f32x16{};
        if (masked) {
          if (fast)
            pair_exact<false, true>(own_p, own_g, dwl, s, dp, ts, hf, g, beta, lt.rel, tsk, bl, NB, lo_row, hi_row);
          else
            pair_exact<true, true>(own_p, own_g, dwl, s, dp, ts, hf, g, beta, lt.rel, tsk, bl, NB, lo_row, hi_row);
        } else {
          const int2 br = ts.blk[hf];  // the plan covers this wave's block only
          const Plan pl = make_plan<-1>(lt.rel, kvalid, br.x, br.y, bl);
          const int mode = wave_mode(pl.n);
          const int32_t* rows = ts.un[pl.flip ? 1 : 0] + hf * 32 + 4 * g;
          blo = pl.blo;
#define HSTU_PLAN(M) pair_plan<M>(own_p, own_g, dw4, s, dp, rows, beta, pl.c0, pl.c1, pl.c2, pl.c3, pl.t1, pl.t2, pl.t3)
          if (mode == kModeConst)
            HSTU_PLAN(kModeConst);
          else if (mode == kModeThr1)
            HSTU_PLAN(kModeThr1);
          else if (mode == kModeThr3)
            HSTU_PLAN(kModeThr3);
          else
            pair_exact<false, false>(own_p, own_g, dwl, s, dp, ts, hf, g, beta, lt.rel, tsk, bl, NB, 0, BQ);
#undef HSTU_PLAN
        }
        xch[wave][0][lane] = own_p[0];
        xch[wave][1][lane] = own_p[1];
        xch[wave][2][lane] = own_g[0];
        xch[wave][3][lane] = own_g[1];
      } else if (g_on) {
        // a block that is not live stores zeros as its G
        xch[wave][2][lane] = u32x4{};
        xch[wave][3][lane] = u32x4{};
      }
      if (nx.valid() && wave == 0) ts_tile_fill<BQ>(sm.ts[cur ^ 1], tsv, nx.nq(), lane, base);
      __syncthreads();
      if (live) {
        contract_half<D>(dvacc, db, ofs, hf, own_p, hf);
        contract_half<D>(dkacc, qb, ofs, hf, own_g, hf);
      }
      if (par_live) {
        const int pw = wave ^ 4;
        const u32x4 par_p[2] = {xch[pw][0][lane], xch[pw][1][lane]};
        const u32x4 par_g[2] = {xch[pw][2][lane], xch[pw][3][lane]};
        contract_half<D>(dvacc, db, ofs, hf, par_p, hf ^ 1);
        contract_half<D>(dkacc, qb, ofs, hf, par_g, hf ^ 1);
      }
      if (g_on && wave < 4) {
        // stored G, written after the products (the loading waves wait for
        // their tile loads here): this wave's 32 keys over the step's 64 rows,
        // its own block (rows 0-31) and its partner's (rows 32-63; zero where a
        // block is not live), into the block of (query tile q0 / kGRows, its
        // key tile).  Re-gathered from the exchange slots so that each lane
        // stores one 16-byte chunk (8 rows of one key) and each key's 64 rows
        // are one 128-byte line: chunk c of key r holds rows 8c .. 8c+7, whose
        // halves sit with lanes (r, g = 0) and (r, g = 1) as run c % 4 of
        // their values (a block that is not live left zeros in its slots).
        // Written once and read once: streamed past the caches.
        const int gi = q0 / kGRows;
        const int64_t gidx = gbase + (int64_t)gi * (gi + 1) + gkt;
        if (gidx < p.g_blocks) {
          char* gb = reinterpret_cast<char*>(p.g) + gidx * kGBlockBytes;
          const int c = lane >> 3, j = c & 3;
          const char* x = reinterpret_cast<const char*>(&xch[c < 4 ? wave : wave ^ 4][2 + (j >> 1)][0]) + 8 * (j & 1);
          // the eight reads issued together (in bounds whether or not the
          // block is live), then the four stores
          u32x2 lo[4], hi[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + (lane & 7);  // key within the wave's 32
            lo[k] = *reinterpret_cast<const u32x2*>(x + 16 * r);
            hi[k] = *reinterpret_cast<const u32x2*>(x + 16 * (r + 32));
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int row = gk0 + 8 * k + (lane & 7), col = q0 % kGRows + 8 * c;
            const u32x4 v = u32x4{lo[k][0], lo[k][1], hi[k][0], hi[k][1]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(gb + (row * kGRows + col) * 2));
          }
        }
      }
      // the next tiles have landed, and every wave is done with this step's
      // tiles and exchange slots, once all waves are here (the loading waves
      // wait for their tile loads; the stored-G writes stay in flight)
      if (loader) wait_loads();
      {
        // d(ts_weights) of a plan step.  Neighbouring keys usually share
        // their first bin, and lanes adding to one LDS address serialise: a
        // 16-lane row whose lanes share it sums its four contributions first
        // (DPP moves) and its first lane adds them, each row to a bin copy of
        // its own; otherwise every lane adds its own four.
        int bmn = blo, bmx = blo;
        row_min_max(bmn, bmx);
        if (bmn == bmx) {
#pragma unroll
          for (int k = 0; k < 4; ++k) dw4[k] = row_sum(dw4[k]);
          if ((lane & 15) == 0) {
            float* dr = dwbins[lane >> 4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (dw4[k] != 0.0f) atomicAdd(&dr[blo + k], dw4[k]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (dw4[k] != 0.0f) atomicAdd(&dwl[blo + k], dw4[k]);
        }
      }
      lds_barrier();
      si = nx;
      cur ^= 1;
    }
    if (kvalid) {
      store_scaled<T, D / 2>(dK + krow * ld + h * D + hf * (D / 2), dkacc, p.alpha, g);
      store_scaled<T, D / 2>(dV + krow * ld + h * D + hf * (D / 2), dvacc, kNegLn2, g);
    }
    __syncthreads();
    for (int i = tid; i < NB; i += NT) {
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < kHalfDwCopies; ++c) v += dwbins[c][i];
      if (v != 0.0f) atomicAdd(p.dw_acc + (int64_t)h * NB + i, p.alpha * v);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major pass: dQ.  Same item list and lane ownership as the
// forward; Sᵀ = K Qᵀ and dPᵀ = V dOᵀ are recomputed and dQᵀ += Kᵀ Gᵀ (K read
// transposed from the same tile).
// ---------------------------------------------------------------------------
namespace {

template <typename T, int D, bool MASK, typename Mid>
__device__ __forceinline__ void q_tile(f32x16* dqacc, const T* kt, const T* vt, const TsTile<BN>& ts,
                                       const TileOps<T, D>& ops, const typename Mma<T>::operand* qop,
                                       const typename Mma<T>::operand* dop, int mode, const Plan& pl,
                                       const FwdLane& ln, const BiasLds& bl, Mid&& mid) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    f32x16 s, dp;
    if constexpr (sizeof(T) == 2) {
      ops.rows2(s, dp, kt, vt, blk, qop, dop);
    } else {
      s = ops.rows(kt, blk, qop);
      dp = ops.rows(vt, blk, dop);
    }
    float cb[16];
    block_bias_mode<+1, BN, false, MASK>(cb, nullptr, mode, pl, ln.tsr, ln.ts64, ts, blk, ln.g, bl, ln.nb);
    float gv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float y = fmaf(s[i], ln.beta, cb[i]);
      const float sg = sigmoid_y(y);
      const float a = y * sg;
      const float u = fmaf(-a, sg, a);
      const float gg = dp[i] * fmaf(u, kNegLn2, sg);
      gv[i] = (MASK && acc_row(i, ln.g) > ln.lim - 32 * blk) ? 0.0f : gg;
    }
    ops.contract(dqacc, kt, gv, blk);
    if (blk == 0) mid();
  }
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_kernel(const AttnParams p) {
  using M = Mma<T>;
  using op_t = typename M::operand;
  if (p.g && p.ctr[kCtrGMode]) return;  // bwd_q_g_kernel does the pass from the stored gradient
  __shared__ KvSmem<T, D> sm;
  __shared__ TsTile<BN> tsm[2];
  __shared__ BiasLds bl;
  __shared__ int item_slot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r32 = lane & 31, g = lane >> 5;
  TileOps<T, D> ops;
  ops.init(lane);
  const int H = p.H, NB = p.NB;
  const int64_t ld = (int64_t)H * D;
  const uint32_t lane_off = tile_lane_offset<T, D, kThreads>(tid, ld);
  const T* Q = static_cast<const T*>(p.q);
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  const T* dO = static_cast<const T*>(p.dout);
  T* dQ = static_cast<T*>(p.dq);
  publish_dw(p, tid);
  load_bucket_tables(bl, p, tid);
  const int n_work = p.ctr[kCtrQTiles] * H;

  for (;;) {
    const int w = pop_item(&item_slot, p.ctr + kCtrQNext2, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.qitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int64_t base = p.ts[seq0];
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
    load_bias_values<T>(bl, p, h, tid);
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};

    const int kv_len = it.pos0 + it.n;
    const int wave_qmin = it.pos0 + wave * 32;
    const T* Kh = K + seq0 * ld + h * D;
    const T* Vh = V + seq0 * ld + h * D;
    const LaneTs lt = lane_ts(tsq, qvalid, base);
    FwdLane ln;
    ln.g = g;
    ln.beta = kNegLog2e * p.alpha;
    ln.nb = NB;
    ln.ts64 = tsq;
    ln.tsr = lt.rel;
    int64_t tsv = 0;
    // the item covers key tiles [it.w0, it.w1) of its causal prefix (all of
    // them unless the tile is split)
    {
      const int k0 = it.w0 * BN, nv0 = min(BN, kv_len - k0);
      issue_kv<T, D>(sm, 0, Kh, Vh, ld, k0, nv0, tid, lane_off);
      if (wave == 0) tsv = p.ts[seq0 + k0 + min(lane, nv0 - 1)];
      if (wave == 0) ts_tile_fill<BN>(tsm[0], tsv, nv0, lane, base);
    }
    wait_loads();
    __syncthreads();
    for (int kt = it.w0; kt < it.w1; ++kt) {
      const int cur = (kt - it.w0) & 1;
      const int key0 = kt * BN;
      const int nvalid = min(BN, kv_len - key0);
      const bool more = kt + 1 < it.w1;
      if (more) {
        // the timestamps first: they are staged half-way through the tile
        // (below), where waiting for them leaves the tile loads in flight
        const int nk0 = key0 + BN, nnv = min(BN, kv_len - nk0);
        if (wave == 0) tsv = p.ts[seq0 + nk0 + min(lane, nnv - 1)];
        __builtin_amdgcn_sched_barrier(0);
        issue_kv<T, D>(sm, cur ^ 1, Kh, Vh, ld, nk0, nnv, tid, lane_off);
      }
      const auto stage = [&] {
        if (more && wave == 0) ts_tile_fill<BN>(tsm[cur ^ 1], tsv, min(BN, kv_len - key0 - BN), lane, base);
      };
      const TsTile<BN>& ts = tsm[cur];
      const int4 hdr = ts.hdr;
      const bool fast = lt.fast && hdr.z == 0;
      ln.lim = qpos - key0;
      if (key0 + BN - 1 > wave_qmin || nvalid < BN || !fast) {
        q_tile<T, D, true>(dqacc, sm.k[cur], sm.v[cur], ts, ops, qop, dop, fast ? kModeLut : kModeWide, Plan{}, ln,
                           bl, stage);
      } else {
        const Plan pl = make_plan<+1>(ln.tsr, qvalid, hdr.x, hdr.y, bl);
        q_tile<T, D, false>(dqacc, sm.k[cur], sm.v[cur], ts, ops, qop, dop, wave_mode(pl.n), pl, ln, bl, stage);
      }
      wait_loads();
      __syncthreads();
    }
    if (qvalid) {
      if (it.slot < 0)
        store_scaled<T, D>(dQ + qrow * ld + h * D, dqacc, p.alpha, g);
      else
        store_row_from_acc<float, D>(p.parts + ((int64_t)it.slot * H + h) * kSplitRows * D + (int64_t)qi * D, dqacc, g);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, query-major pass from stored score gradients (bf16, d >= 64,
// cp_size 1): dQᵀ += Kᵀ Gᵀ with G read from the blocks the dK/dV pass wrote,
// so S, dP, the bias and the SiLU gradient are not recomputed.  Same items as
// the forward (query tiles of 128 rows, one per kGRows block column); per key
// tile, the K tile and the G block (row-major) are loaded into swizzled LDS
// tiles (double-buffered) and
// both operands are taken with transpose reads: Kᵀ (d x keys) from the K tile
// and Gᵀ (keys x the wave's 32 rows) from the G tile, in the same key order.
// Masked pairs and rows past a sequence's end hold zero G.
// ---------------------------------------------------------------------------
namespace {

template <int D> struct alignas(16) QgSmem {
  __bf16 k[2][BN * D];
  __bf16 g[2][kGKeys * kGRows];
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_g_kernel(const AttnParams p) {
  using T = __bf16;
  using Ptr = __attribute__((address_space(3))) s16x4*;
  static_assert(BN == kGKeys && BM == kGRows, "one stored-G block per key tile of a query tile");
  if (!p.ctr[kCtrGMode]) return;  // the schedule's shares are not aligned: bwd_q_kernel does the pass
  __shared__ QgSmem<D> sm;
  __shared__ int item_slot;
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  LaneOffsets<D> lk;       // transpose reads of the K tile
  lk.init(lane);
  // transpose reads of the G tile: this wave's column block (its 32 rows)
  int gtr[2];
  {
    using S = SwTile<__bf16, kGRows>;
    const int m = lane & 15, qq = lane >> 4;
    const int rb = 4 * g + (m >> 2), cb = 16 * (qq & 1) + 4 * (m & 3);
    gtr[0] = 2 * S::off(rb, wave * 32 + cb);
    gtr[1] = 2 * S::off(rb + 8, wave * 32 + cb);
  }
  const int H = p.H;
  const int64_t ld = (int64_t)H * D;
  const uint32_t lane_off = tile_lane_offset<T, D, kThreads>(tid, ld);
  const uint32_t g_lane_off = tile_lane_offset<T, kGRows, kThreads>(tid, kGRows);
  const T* K = static_cast<const T*>(p.k);
  T* dQ = static_cast<T*>(p.dq);
  const T* G = reinterpret_cast<const T*>(p.g);
  publish_dw(p, tid);
  const int n_work = p.ctr[kCtrQTiles] * H;

  for (;;) {
    const int w = pop_item(&item_slot, p.ctr + kCtrQNext2, tid);
    if (w >= n_work) break;
    const int h = w % H;
    const Item it = p.qitems[w / H];
    const int64_t seq0 = p.offsets[it.b];
    const int qi = wave * 32 + r32;
    const bool qvalid = qi < it.n;
    const int64_t qrow = (int64_t)it.row0 + qi;
    const int64_t nt = (p.offsets[it.b + 1] - seq0 + kGRows - 1) / kGRows;
    const int gi = it.pos0 / kGRows;
    const int64_t gbase = p.gblk_off[it.b] + h * nt * (nt + 1) + (int64_t)gi * (gi + 1);
    const int kv_len = it.pos0 + it.n;
    const T* Kh = K + seq0 * ld + h * D;
    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};
    // a block outside the allocation (a length past max_seq_len) is never read
    const auto g_ok = [&](int kt) { return gbase + kt < p.g_blocks; };
    // the item covers key tiles [it.w0, it.w1) of its causal prefix (all of
    // them unless the tile is split)
    tile_load_async<T, D, BN, kThreads>(sm.k[0], Kh + (int64_t)it.w0 * BN * ld, ld, min(BN, kv_len - it.w0 * BN), tid,
                                        lane_off);
    if (g_ok(it.w0))
      tile_load_async<T, kGRows, kGKeys, kThreads, 2>(sm.g[0], G + (gbase + it.w0) * (kGKeys * kGRows), kGRows, kGKeys,
                                                   tid, g_lane_off);
    wait_loads();
    __syncthreads();
    for (int kt = it.w0; kt < it.w1; ++kt) {
      const int cur = (kt - it.w0) & 1;
      if (kt + 1 < it.w1) {
        tile_load_async<T, D, BN, kThreads>(sm.k[cur ^ 1], Kh + (int64_t)(kt + 1) * BN * ld, ld,
                                            min(BN, kv_len - (kt + 1) * BN), tid, lane_off);
        if (g_ok(kt + 1))
          tile_load_async<T, kGRows, kGKeys, kThreads, 2>(sm.g[cur ^ 1], G + (gbase + kt + 1) * (kGKeys * kGRows),
                                                       kGRows, kGKeys, tid, g_lane_off);
      }
      if (g_ok(kt)) {
        const char* kb = reinterpret_cast<const char*>(sm.k[cur]);
        const char* gb = reinterpret_cast<const char*>(sm.g[cur]);
        // the G operands of the tile (this wave's 32 rows), then the products
        bf16x8 bg[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int blk = n >> 1, u = n & 1;
          const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Ptr)(gb + gtr[0] + (blk * 32 + 16 * u) * kGRows * 2));
          const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Ptr)(gb + gtr[1] + (blk * 32 + 16 * u) * kGRows * 2));
          const short __attribute__((ext_vector_type(8))) b = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          bg[n] = __builtin_bit_cast(bf16x8, b);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int blk = n >> 1, u = n & 1;
#pragma unroll
          for (int dblk = 0; dblk < D / 32; ++dblk) {
            const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Ptr)(kb + lk.tr[dblk][0] + (blk * 32 + 16 * u) * D * 2));
            const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((Ptr)(kb + lk.tr[dblk][1] + (blk * 32 + 16 * u) * D * 2));
            const short __attribute__((ext_vector_type(8))) a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            dqacc[dblk] = Mma<__bf16>::mma(__builtin_bit_cast(bf16x8, a), bg[n], dqacc[dblk]);
          }
        }
      }
      wait_loads();
      __syncthreads();
    }
    if (qvalid) {
      if (it.slot < 0)
        store_scaled<T, D>(dQ + qrow * ld + h * D, dqacc, p.alpha, g);
      else
        store_row_from_acc<float, D>(p.parts + ((int64_t)it.slot * H + h) * kSplitRows * D + (int64_t)qi * D, dqacc, g);
    }
  }
}

// ---------------------------------------------------------------------------
// Sum of the parts of split query tiles.  A tile whose key walk was split
// over several items has fp32 partial sums in consecutive slots; one
// workgroup per (split tile, head) adds them in part order (so the result
// does not depend on the order the parts ran in), scales and stores the rows.
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_parts_kernel(const float* __restrict__ parts,
                                                                      const SplitTile* __restrict__ splits,
                                                                      const int* __restrict__ ctr,
                                                                      T* __restrict__ out, int H, float scale) {
  constexpr int kVec = D / 4;                                   // float4 per row
  constexpr int kPer = kSplitRows * kVec / kReduceThreads;      // float4 per thread
  static_assert(kPer * kReduceThreads == kSplitRows * kVec, "whole rows per workgroup");
  const int idx = blockIdx.x;
  if (idx >= ctr[kCtrSplits] * H) return;
  const int h = idx % H;
  const SplitTile st = splits[idx / H];
  const int64_t ld = (int64_t)H * D;
  const int nv = st.n * kVec;  // float4 of the tile's rows (a slot is [kSplitRows][D], rows >= n unused)
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < st.nparts; ++k) {
    // all of this part's loads in flight at once, then the adds (part order
    // kept: the sum does not depend on which part ran when)
    const v4f* src = reinterpret_cast<const v4f*>(parts + ((int64_t)(st.slot0 + k) * H + h) * kSplitRows * D);
    v4f x[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = threadIdx.x + i * kReduceThreads;
      x[i] = v < nv ? __builtin_nontemporal_load(src + v) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] += x[i];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = threadIdx.x + i * kReduceThreads;
    if (v >= nv) continue;
    const int r = v / kVec, c = (v % kVec) * 4;
    T* dst = out + (int64_t)(st.row0 + r) * ld + h * D + c;
    const v4f a = acc[i];
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(a.x * scale, a.y * scale), pack_bf16x2(a.z * scale, a.w * scale)};
    } else {
      *reinterpret_cast<float4*>(dst) = float4{a.x * scale, a.y * scale, a.z * scale, a.w * scale};
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {
template <typename K>
int grid_for(K kernel, int max_items, int cus, int threads = kThreads) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
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
    if constexpr (sizeof(T) == 2 && D >= 64) {
      auto k = bwd_kv_half_kernel<D>;
      hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus, kHalfThreads)), dim3(kHalfThreads), 0, s, p);
    } else {
      auto k = bwd_kv_kernel<T, D>;
      hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus)), dim3(kThreads), 0, s, p);
    }
  } else {
    if constexpr (sizeof(T) == 2 && D >= 64) {
      if (p.g) {
        // the scheduler decides on the device whether the stored gradient
        // applies (ctr[kCtrGMode]); a context-parallel share launches both
        // passes and the one that does not apply returns at once (without
        // context parallelism it always applies)
        auto k = bwd_q_g_kernel<D>;
        hipLaunchKernelGGL(k, dim3(grid_for(k, max_items, cus)), dim3(kThreads), 0, s, p);
        if (p.cp_size == 1) return hipGetLastError();
      }
    }
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

namespace {
template <typename T, int D>
hipError_t launch_reduce_t(const AttnParams& p, int which, int max_splits, hipStream_t s) {
  T* out = static_cast<T*>(which == 0 ? p.out : p.dq);
  const float scale = which == 0 ? kNegLn2 : p.alpha;
  hipLaunchKernelGGL((reduce_parts_kernel<T, D>), dim3(max_splits * p.H), dim3(kReduceThreads), 0, s, p.parts,
                     p.splits, p.ctr, out, p.H, scale);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_d(const AttnParams& p, int d, int which, int max_splits, hipStream_t s) {
  switch (d) {
    case 32: return launch_reduce_t<T, 32>(p, which, max_splits, s);
    case 64: return launch_reduce_t<T, 64>(p, which, max_splits, s);
    case 128: return launch_reduce_t<T, 128>(p, which, max_splits, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_reduce(const AttnParams& p, bool bf16, int d, int which, int max_splits, hipStream_t s) {
  if (max_splits <= 0 || !p.parts) return hipSuccess;
  return bf16 ? launch_reduce_d<__bf16>(p, d, which, max_splits, s) : launch_reduce_d<float>(p, d, which, max_splits, s);
}

int attn_q_tile_rows() { return BM; }
int attn_k_tile_keys() { return BN; }
int attn_bwd_key_tile(bool bf16, int d) { return bf16 && d >= 64 ? kHalfKeys : BK; }
int attn_bwd_q_step() { return BQ; }

}  // namespace hstu
