// Timestamp-bias selection for a score tile (Scaling Generative Recommendations
// with Context Parallelism on HSTU, §2.1, timestamp-bias paragraph).
//
// Every lane of the attention kernels owns one row r (a query in the forward
// and dQ passes, a key in the dK/dV pass) and computes, per tile, the scores of
// its row against the tile's "other" rows o.  The bucket of a pair depends on
// Δ = ts_query - ts_key, i.e. Δ = σ (ts_r - ts_o) with σ = +1 when the lane owns
// the query and σ = -1 when it owns the key.
//
// Exact bucket.  bucket(m) = #{k in [1, NB) : m >= E_k} for m = |Δ|.  An
// integer m >= 1 falls in octave e = floor(log2 m) and, within it, in one of 32
// sub-bins given by the five bits after the leading one.  For NB <= 512 a
// sub-bin never holds two edges (edges are at least 2^(1/16) apart, a sub-bin
// spans at most a factor 33/32), so a 1024-entry table of pairs {E, b} with
// bucket(m) = b + [m >= E] gives the bucket with one lookup and one compare
// (E is the edge inside the sub-bin, or 0 with b one below the sub-bin's
// bucket when it holds none).  The table is indexed by the leading-zero count
// z = 31 - e, so the index is (z << 5) | sub-bin.
//
// Tile plans.  The bucket is a monotone step function of |Δ|.  In an unmasked
// tile every lane sees all rows of the tile, so the range of Δ over the tile
// follows from the tile's timestamp range and the lane's own timestamp.  If
// that range keeps one sign and crosses n <= 3 bucket edges, the bias of an
// element is chosen by n compares of a 32-bit timestamp offset against
// per-lane thresholds (the edges are nested, so the compares chain).  The wave
// takes the largest n of its lanes (uniform branches); otherwise the exact
// bucket is looked up per element.
#pragma once

#include "common.h"

namespace hstu {

constexpr int kLutSize = 1024;
constexpr int kModeConst = 0, kModeThr1 = 1, kModeThr3 = 3, kModeLut = 4, kModeWide = 5;

// Bias tables of one work item, in LDS.  e and c are padded past NB so that
// plan lookups at b_lo + 3 need no clamping.
constexpr int kPad = 4;
struct alignas(16) BiasLds {
  u32x2 lut[kLutSize];              // {E, b}: bucket(m) = b + [m >= E]
  int32_t e[kMaxBuckets + kPad];    // min(E_k, 2^31 - 1), k = 0..NB; 2^31 - 1 past NB
  float c[kMaxBuckets + kPad];      // -log2(e) * alpha * w[h, b]; padded with c[NB - 1]
};

__device__ __forceinline__ int lut_bucket(uint32_t m, const u32x2* __restrict__ lut) {
  m = m > 1u ? m : 1u;  // buckets of 0 and 1 agree (E_1 >= 2)
  const int z = __builtin_clz(m);
  const uint32_t t = m << z;
  const u32x2 L = lut[(z << 5) | (int)((t >> 26) & 31u)];
  return (int)L.y + (m >= L.x ? 1 : 0);
}

__device__ __forceinline__ int lut_bucket64(int64_t d, int nb, const u32x2* __restrict__ lut) {
  const uint64_t m = d < 0 ? (uint64_t)(-d) : (uint64_t)d;
  return (m >> 32) ? nb - 1 : lut_bucket((uint32_t)m, lut);
}

// Timestamps of the tile's other rows, staged in LDS by one wave, relative to
// the base of the work item (the first timestamp of its sequence).  Rows past
// the last valid one repeat its timestamp.  u = ts - base and nu = ~u (for
// compares whose direction is flipped), held as un[0] and un[1] so that a
// flip selects by index; hdr = {min u, max u, wide, 0} over the tile and
// blk[b] = {min u, max u} over its 32-row block b.
template <int N> struct alignas(16) TsTile {
  int32_t un[2][N];
  int64_t t64[N];
  int4 hdr;  // wide: some |ts - base| is 2^30 or more, only the 64-bit path is exact
  int2 blk[N / 32];
};

// Min and max over each 16-lane row, left in every lane of the row: two
// quad permutations, then the half-row and row mirrors (DPP moves, no LDS
// round trip).
__device__ __forceinline__ void row_min_max(int32_t& mn, int32_t& mx) {
  int32_t a = __builtin_amdgcn_update_dpp(0, mn, 0xB1, 0xF, 0xF, false);  // lane ^ 1
  int32_t b = __builtin_amdgcn_update_dpp(0, mx, 0xB1, 0xF, 0xF, false);
  mn = min(mn, a);
  mx = max(mx, b);
  a = __builtin_amdgcn_update_dpp(0, mn, 0x4E, 0xF, 0xF, false);  // lane ^ 2
  b = __builtin_amdgcn_update_dpp(0, mx, 0x4E, 0xF, 0xF, false);
  mn = min(mn, a);
  mx = max(mx, b);
  a = __builtin_amdgcn_update_dpp(0, mn, 0x141, 0xF, 0xF, false);  // lane 7 - i within 8 lanes
  b = __builtin_amdgcn_update_dpp(0, mx, 0x141, 0xF, 0xF, false);
  mn = min(mn, a);
  mx = max(mx, b);
  a = __builtin_amdgcn_update_dpp(0, mn, 0x140, 0xF, 0xF, false);  // lane 15 - i within the row
  b = __builtin_amdgcn_update_dpp(0, mx, 0x140, 0xF, 0xF, false);
  mn = min(mn, a);
  mx = max(mx, b);
}

// Sum over each 16-lane row, the same value left in every lane of the row
// (the moves pair lanes symmetrically, so every lane adds the same operands).
__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Filled by one wave: lane j holds the timestamp of row j; rows >= nvalid
// (nvalid >= 1, the same in every lane) are invalid.  The ranges are reduced
// with row-local DPP moves and four lane reads, so the staging costs no LDS
// round trips of its own.
template <int N>
__device__ __forceinline__ void ts_tile_fill(TsTile<N>& t, int64_t ts, int nvalid, int lane, int64_t base) {
  static_assert(N == 64, "one wave fills the tile");
  const int src = __builtin_amdgcn_readfirstlane(nvalid - 1);
  const uint64_t tsu = (uint64_t)ts;
  const uint32_t last_lo = __builtin_amdgcn_readlane((uint32_t)tsu, src);
  const uint32_t last_hi = __builtin_amdgcn_readlane((uint32_t)(tsu >> 32), src);
  const int64_t last = (int64_t)(((uint64_t)last_hi << 32) | last_lo);
  const int64_t v = lane < nvalid ? ts : last;
  const int64_t rel = v - base;
  const bool wide = __ballot(rel <= -(1ll << 30) || rel >= (1ll << 30)) != 0;
  const int32_t r32 = wide ? 0 : (int32_t)rel;
  int32_t mn = r32, mx = r32;
  row_min_max(mn, mx);
  const int32_t n0 = __builtin_amdgcn_readlane(mn, 0), n1 = __builtin_amdgcn_readlane(mn, 16);
  const int32_t n2 = __builtin_amdgcn_readlane(mn, 32), n3 = __builtin_amdgcn_readlane(mn, 48);
  const int32_t x0 = __builtin_amdgcn_readlane(mx, 0), x1 = __builtin_amdgcn_readlane(mx, 16);
  const int32_t x2 = __builtin_amdgcn_readlane(mx, 32), x3 = __builtin_amdgcn_readlane(mx, 48);
  t.un[0][lane] = r32;
  t.un[1][lane] = ~r32;
  t.t64[lane] = v;
  if (lane == 0) {
    // the range of each 32-row half, and of the tile
    const int32_t b0n = min(n0, n1), b0x = max(x0, x1), b1n = min(n2, n3), b1x = max(x2, x3);
    t.blk[0] = int2{b0n, b0x};
    t.blk[1] = int2{b1n, b1x};
    t.hdr = int4{min(b0n, b1n), max(b0x, b1x), wide ? 1 : 0, 0};
  }
}

// Per-lane plan of an unmasked tile.
struct Plan {
  float c0, c1, c2, c3;  // c[b_lo + k]
  int32_t t1, t2, t3;    // element passes edge b_lo + k iff v <= t_k
  int flip;              // v = nu instead of u
  int n;                 // edges crossed, or kModeLut
  int blo;               // bucket of the smallest |Δ| (0 for invalid lanes)
};

// tsr: the lane's timestamp minus the item base (|tsr| < 2^30); [tlo, thi]:
// the tile's range of u.  Invalid lanes get n = 0.  Thresholds of edges past
// the ones the tile crosses are never passed (those edges exceed every |Δ| of
// the tile), so all three are set unconditionally; a threshold below the
// int32 range saturates, which also never passes (|u| < 2^30).
template <int SIGMA>
__device__ __forceinline__ Plan make_plan(int32_t tsr, bool valid, int32_t tlo, int32_t thi, const BiasLds& bl) {
  const int32_t dmin = SIGMA > 0 ? tsr - thi : tlo - tsr;
  const int32_t dmax = SIGMA > 0 ? tsr - tlo : thi - tsr;
  const bool pos = dmin >= 0, neg = dmax <= 0;
  const uint32_t mlo = (uint32_t)(pos ? dmin : -dmax);
  const uint32_t mhi = (uint32_t)(pos ? dmax : -dmin);
  const int blo = lut_bucket(mlo, bl.lut);
  const int bhi = lut_bucket(mhi, bl.lut);
  const int n = !valid ? 0 : ((pos || neg) ? bhi - blo : kModeLut);
  // |Δ| >= E:  kappa = +1: u <= tsr - E;  kappa = -1: u >= tsr + E, i.e. ~u <= ~tsr - E.
  const bool kpos = pos ? SIGMA > 0 : SIGMA < 0;
  const int32_t R = kpos ? tsr : ~tsr;
  const int b0 = valid ? blo : 0;
  Plan p;
  p.n = n > 3 ? kModeLut : n;
  p.flip = kpos ? 0 : 1;
  p.blo = b0;
  p.c0 = bl.c[b0];
  p.c1 = bl.c[b0 + 1];
  p.c2 = bl.c[b0 + 2];
  p.c3 = bl.c[b0 + 3];
  p.t1 = __builtin_elementwise_sub_sat(R, bl.e[b0 + 1]);
  p.t2 = __builtin_elementwise_sub_sat(R, bl.e[b0 + 2]);
  p.t3 = __builtin_elementwise_sub_sat(R, bl.e[b0 + 3]);
  return p;
}

// Wave mode of an unmasked tile from the lanes' plans.
__device__ __forceinline__ int wave_mode(int n) {
  if (__ballot(n > 3)) return kModeLut;
  if (__ballot(n >= 2)) return kModeThr3;
  if (__ballot(n == 1)) return kModeThr1;
  return kModeConst;
}

// Other-row values of one 32-row block for this lane: value i belongs to row
// blk*32 + acc_row(i, g), i.e. four runs of four consecutive rows.
__device__ __forceinline__ void block_rows_i32(int32_t* v, const int32_t* __restrict__ arr, int blk, int g) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int4 x = *reinterpret_cast<const int4*>(arr + blk * 32 + q4 * 8 + 4 * g);
    v[4 * q4 + 0] = x.x;
    v[4 * q4 + 1] = x.y;
    v[4 * q4 + 2] = x.z;
    v[4 * q4 + 3] = x.w;
  }
}

// Bias values of one 32-row block: cb[i] for the row blk*32 + acc_row(i, g).
// With KEYS, key[i] receives the number of plan edges the element passes
// (plan modes) or its bucket (exact modes).  kModeConst/Thr1/Thr3 use the
// plan; kModeLut needs |tsr| < 2^30 and a tile that is not wide; kModeWide is
// exact for any timestamps.  The plan's fields arrive as separate scalars: a
// chain of selects between fields of one struct would otherwise be turned into
// an indexed load from a stack copy of it.
template <int MODE, int SIGMA, int N, bool KEYS>
__device__ __forceinline__ void block_bias(float* cb, int* key, float c0, float c1, float c2, float c3, int32_t t1,
                                           int32_t t2, int32_t t3, int flip, int32_t tsr, int64_t tsr64,
                                           const TsTile<N>& t, int blk, int g, const BiasLds& bl, int nb) {
  int32_t v[16];
  if constexpr (MODE == kModeConst) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cb[i] = c0;
      if constexpr (KEYS) key[i] = 0;
    }
  } else if constexpr (MODE == kModeThr1 || MODE == kModeThr3) {
    block_rows_i32(v, flip ? t.un[1] : t.un[0], blk, g);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool p1 = v[i] <= t1;
      float c = p1 ? c1 : c0;
      int k = p1 ? 1 : 0;
      if constexpr (MODE == kModeThr3) {
        const bool p2 = v[i] <= t2, p3 = v[i] <= t3;
        c = p2 ? c2 : c;
        c = p3 ? c3 : c;
        k += (p2 ? 1 : 0) + (p3 ? 1 : 0);
      }
      cb[i] = c;
      if constexpr (KEYS) key[i] = k;
    }
  } else if constexpr (MODE == kModeLut) {
    block_rows_i32(v, t.un[0], blk, g);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t d = SIGMA > 0 ? tsr - v[i] : v[i] - tsr;
      const int b = lut_bucket((uint32_t)(d < 0 ? -d : d), bl.lut);
      cb[i] = bl.c[b];
      if constexpr (KEYS) key[i] = b;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t o = t.t64[blk * 32 + acc_row(i, g)];
      const int b = lut_bucket64(SIGMA > 0 ? tsr64 - o : o - tsr64, nb, bl.lut);
      cb[i] = bl.c[b];
      if constexpr (KEYS) key[i] = b;
    }
  }
}

// Bias of one block under a wave-uniform mode (plan fields passed on as
// scalars).  Masked tiles only use the exact modes.
template <int SIGMA, int N, bool KEYS, bool EXACT_ONLY>
__device__ __forceinline__ void block_bias_mode(float* cb, int* key, int mode, const Plan& pl, int32_t tsr,
                                                int64_t tsr64, const TsTile<N>& t, int blk, int g, const BiasLds& bl,
                                                int nb) {
#define HSTU_BIAS(M)                                                                                            \
  block_bias<M, SIGMA, N, KEYS>(cb, key, pl.c0, pl.c1, pl.c2, pl.c3, pl.t1, pl.t2, pl.t3, pl.flip, tsr, tsr64, t, \
                                blk, g, bl, nb)
  if (mode == kModeWide) {
    HSTU_BIAS(kModeWide);
  } else if (EXACT_ONLY || mode == kModeLut) {
    HSTU_BIAS(kModeLut);
  } else if (mode == kModeConst) {
    HSTU_BIAS(kModeConst);
  } else if (mode == kModeThr1) {
    HSTU_BIAS(kModeThr1);
  } else {
    HSTU_BIAS(kModeThr3);
  }
#undef HSTU_BIAS
}

}  // namespace hstu
