// Timestamp-bias selection for a score tile.
//
// Every lane of the attention kernels owns one row r (a query in the forward
// and dQ passes, a key in the dK/dV pass) and computes, per tile, the scores of
// its row against the tile's "other" rows o.  The bucket of a pair depends on
// Δ = ts_query - ts_key (Scaling Generative Recommendations with Context
// Parallelism on HSTU, §2.1, timestamp-bias paragraph), i.e. Δ = σ (ts_r - ts_o)
// with σ = +1 when the lane owns the query and σ = -1 when it owns the key.
//
// The bucket is a monotone step function of |Δ|.  So, per lane and tile, the
// range of Δ over the other rows the lane can actually see (causal mask)
// bounds the buckets it can meet.  If that range crosses n <= 3 bucket edges
// (and keeps one sign), the bucket of an element is b_lo plus the number of
// edges it passes, and passing edge t is one compare of the element's 32-bit
// timestamp offset against a per-lane threshold; the edges are nested, so the
// bias is a chain of selects.  Otherwise (n > 3, a sign change, or timestamps
// spread too wide for 32-bit offsets) the exact bucket is computed per element.
// The wave takes the largest n of its lanes, so branches stay uniform.
#pragma once

#include "common.h"

namespace hstu {

constexpr int kMaxEdges = 3;   // threshold compares per element before the exact path
constexpr int kModeExact = kMaxEdges + 1;

// Timestamps of the tile's other rows, staged in LDS.  Rows past the last
// valid one repeat its timestamp.  The range of timestamps a lane sees is a
// prefix (rows 0..j: the lane owns a query and sees keys up to its position)
// or a suffix (rows j..N-1: the lane owns a key, seen by queries from its
// position on).  For non-decreasing timestamps (the usual case, flagged
// `sorted`) the range is read off t64 directly; otherwise `lo`/`hi` hold the
// running minima/maxima.
template <int N> struct alignas(16) TsTile {
  int64_t t64[N];
  int64_t lo[N];
  int64_t hi[N];
  int32_t t32[N];   // t64 - base (valid when !wide)
  int64_t base;
  int wide;         // some |t64 - base| is 2^30 or more
  int sorted;       // t64 is non-decreasing
};

// Filled by one wave (N == 64): lane j holds the timestamp of row j; rows
// >= nvalid (nvalid >= 1) are invalid.
template <int N, bool SUFFIX>
__device__ __forceinline__ void ts_tile_fill(TsTile<N>& t, int64_t ts, int nvalid, int lane) {
  static_assert(N == 64, "one wave fills the tile");
  const int64_t last = __shfl(ts, nvalid - 1);
  const int64_t v = lane < nvalid ? ts : last;
  const int64_t prev = __shfl_up(v, 1);
  const bool sorted = __ballot(lane > 0 && v < prev) == 0;
  const int64_t base = __shfl(v, 0);
  const int64_t rel = v - base;
  const bool wide = __ballot(rel <= -(1ll << 30) || rel >= (1ll << 30)) != 0;
  t.t64[lane] = v;
  t.t32[lane] = wide ? 0 : (int32_t)rel;
  if (!sorted) {
    int64_t vmin = v, vmax = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t omin = SUFFIX ? __shfl_down(vmin, off) : __shfl_up(vmin, off);
      const int64_t omax = SUFFIX ? __shfl_down(vmax, off) : __shfl_up(vmax, off);
      const bool in = SUFFIX ? (lane + off < 64) : (lane >= off);
      if (in) {
        vmin = omin < vmin ? omin : vmin;
        vmax = omax > vmax ? omax : vmax;
      }
    }
    t.lo[lane] = vmin;
    t.hi[lane] = vmax;
  }
  if (lane == 0) {
    t.base = base;
    t.wide = wide ? 1 : 0;
    t.sorted = sorted ? 1 : 0;
  }
}

// Range of timestamps over rows [a, b] of the tile (a <= b): a prefix range
// (a == 0) for SUFFIX == false, a suffix range (b == N-1) for SUFFIX == true.
template <int N, bool SUFFIX>
__device__ __forceinline__ void ts_tile_range(const TsTile<N>& t, int a, int b, int64_t* tmin, int64_t* tmax) {
  if (t.sorted) {
    *tmin = t.t64[a];
    *tmax = t.t64[b];
  } else {
    const int j = SUFFIX ? a : b;
    *tmin = t.lo[j];
    *tmax = t.hi[j];
  }
}

struct LaneBias {
  float c0, c1, c2, c3;     // alpha * w[b_lo + k], k = 0..3
  int32_t t0, t1, t2;       // element passes edge k iff (t32 <= t_k) != flip
  int32_t flip;
  int b_lo;
  int n;                    // edges crossed (0..kMaxEdges) or kModeExact
};

__device__ __forceinline__ int32_t clamp_i32(int64_t x) {
  return (int32_t)(x > 2147483647ll ? 2147483647ll : (x < -2147483647ll - 1 ? -2147483647ll - 1 : x));
}

// Per-lane bias plan.  tsr: the lane's own timestamp; [tmin, tmax]: range of
// the other rows it sees (any == false: it sees none, everything is masked).
// Scalar fields and one exit keep the plan in registers.
template <int SIGMA>
__device__ __forceinline__ LaneBias lane_bias(int64_t tsr, int64_t tmin, int64_t tmax, bool any, int64_t base,
                                              int wide, const float* __restrict__ wtab,
                                              const u32x2* __restrict__ ep, int nb, float nb32) {
  const int64_t dmin = SIGMA > 0 ? tsr - tmax : tmin - tsr;
  const int64_t dmax = SIGMA > 0 ? tsr - tmin : tmax - tsr;
  const bool pos = dmin >= 0, neg = dmax <= 0;
  const int dir = pos ? 0 : 1;
  const int64_t mlo = pos ? dmin : -dmax;
  const int64_t mhi = pos ? dmax : -dmin;
  const int blo = bucket_of(mlo, nb, nb32, ep);
  const int bhi = bucket_of(mhi, nb, nb32, ep);
  const int n = bhi - blo;
  const bool exact = any && ((!pos && !neg) || n > kMaxEdges || (n > 0 && wide));
  // Element |Δ| >= E passes the edge.  With Δ = σ(tsr - tso):
  //   σ(tsr - tso) >= E  (dir 0) / -σ(tsr - tso) >= E  (dir 1)
  // reduces to tso <= tsr - E (flip 0) or tso >= tsr + E, i.e. !(tso <= tsr + E - 1) (flip 1).
  const int flip = (any && !exact) ? (SIGMA > 0 ? dir : 1 - dir) : 0;
  const int nn = (any && !exact) ? n : 0;
  const int32_t never = flip ? INT32_MAX : INT32_MIN;
  const int b0 = any && !exact ? blo : 0;
  auto thr = [&](int k) -> int32_t {
    if (k >= nn) return never;
    const int64_t E = (int64_t)ep[b0 + k + 1].x;
    return clamp_i32((flip ? tsr + E - 1 : tsr - E) - base);
  };
  LaneBias r;
  r.b_lo = b0;
  r.n = exact ? kModeExact : nn;
  r.flip = flip;
  r.c0 = any ? wtab[b0] : 0.0f;
  r.c1 = any ? wtab[min(b0 + 1, nb - 1)] : 0.0f;
  r.c2 = any ? wtab[min(b0 + 2, nb - 1)] : 0.0f;
  r.c3 = any ? wtab[min(b0 + 3, nb - 1)] : 0.0f;
  r.t0 = thr(0);
  r.t1 = thr(1);
  r.t2 = thr(2);
  return r;
}

// Bias values cb[i] for the 16 accumulator values of one 32-row block of the
// tile (rows blk*32 + acc_row(i, g)) under wave mode `nw` (the largest n of the
// wave's lanes).  bsel[i] receives the number of edges passed (threshold modes)
// or the exact bucket (exact mode).  In exact mode, when every lane of the wave
// has |tsr - base| < 2^30 (fast32) and the tile is not wide, |Δ| < 2^31 is
// formed from 32-bit offsets.
template <int SIGMA, int N>
__device__ __forceinline__ void block_bias(float* cb, int* bsel, int nw, const LaneBias lb, int64_t tsr,
                                           int32_t tsr_rel, bool fast32, const TsTile<N>& t, int blk, int g,
                                           const float* __restrict__ wtab, const u32x2* __restrict__ ep, int nb,
                                           float nb32) {
  if (nw == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cb[i] = lb.c0;
      bsel[i] = 0;
    }
  } else if (nw <= kMaxEdges) {
    const bool fl = lb.flip != 0;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int j0 = blk * 32 + q4 * 8 + 4 * g;
      const int4 v = *reinterpret_cast<const int4*>(&t.t32[j0]);
      const int32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool p0 = (vv[u] <= lb.t0) != fl;
        const bool p1 = (vv[u] <= lb.t1) != fl;
        const bool p2 = (vv[u] <= lb.t2) != fl;
        cb[q4 * 4 + u] = p2 ? lb.c3 : (p1 ? lb.c2 : (p0 ? lb.c1 : lb.c0));
        bsel[q4 * 4 + u] = (int)p0 + (int)p1 + (int)p2;
      }
    }
  } else if (fast32) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int j0 = blk * 32 + q4 * 8 + 4 * g;
      const int4 v = *reinterpret_cast<const int4*>(&t.t32[j0]);
      const int32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int32_t d = SIGMA > 0 ? tsr_rel - vv[u] : vv[u] - tsr_rel;
        const int b = bucket_u32((uint32_t)(d < 0 ? -d : d), nb, nb32, ep);
        cb[q4 * 4 + u] = wtab[b];
        bsel[q4 * 4 + u] = b;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = blk * 32 + acc_row(i, g);
      const int64_t d = SIGMA > 0 ? tsr - t.t64[j] : t.t64[j] - tsr;
      const int b = bucket_of(d, nb, nb32, ep);
      cb[i] = wtab[b];
      bsel[i] = b;
    }
  }
}

// Whether the lane's own timestamp is close enough to the tile base for the
// 32-bit exact path (wave-uniform result).
__device__ __forceinline__ bool wave_fast32(int64_t tsr, int64_t base, int wide, int32_t* rel) {
  const int64_t d = tsr - base;
  const bool ok = d > -(1ll << 30) && d < (1ll << 30);
  *rel = ok ? (int32_t)d : 0;
  return !wide && __ballot(!ok) == 0;
}

// Largest n over the wave's lanes.
__device__ __forceinline__ int wave_mode(int n) {
  if (__ballot(n == kModeExact)) return kModeExact;
  if (__ballot(n == 3)) return 3;
  if (__ballot(n == 2)) return 2;
  if (__ballot(n == 1)) return 1;
  return 0;
}

}  // namespace hstu
