// Jagged tile scheduler (one workgroup).  From the int64 offsets it builds
//   - the rank-local query offsets (context-parallel share: chunks r and
//     2C-1-r of every sequence; Scaling Generative Recommendations with Context
//     Parallelism on HSTU, §2.3, load-balanced mini-chunks),
//   - the list of query tiles and the list of key tiles, each sorted by
//     descending cost with a counting sort, so that persistent workgroups that
//     pop items in order take the longest work first,
// and resets the work counters.  Tiles lying entirely above the causal
// diagonal are never emitted: a query tile's key range stops at its last row.
#include <mutex>

#include "attn.h"
#include "bias.h"

namespace hstu {

namespace {

constexpr int kSchedThreads = 1024;

// Candidates of sequence b (length L), clamped to [0, L]; none without a list.
__device__ __forceinline__ int candidates(const int64_t* num_targets, int b, int L) {
  if (!num_targets) return 0;
  const int64_t m = num_targets[b];
  return (int)(m < 0 ? 0 : (m > L ? L : m));
}

struct SegInfo {
  int n;
  int pos0[2];
  int len[2];
  int64_t lrow0[2];
};

__device__ __forceinline__ int chunk_lo(int64_t L, int k, int nch) { return (int)((int64_t)k * L / nch); }

__device__ __forceinline__ SegInfo seq_segments(const SchedParams& p, int b, int64_t local0) {
  const int64_t o0 = p.offsets[b];
  const int L = (int)(p.offsets[b + 1] - o0);
  SegInfo s;
  if (p.targets_only) {  // the query rows are the candidates, the last num_targets[b] positions
    const int m = candidates(p.num_targets, b, L);
    s.n = 1;
    s.pos0[0] = L - m;
    s.len[0] = m;
    s.lrow0[0] = local0;
    return s;
  }
  if (p.cp_size == 1) {
    s.n = 1;
    s.pos0[0] = 0;
    s.len[0] = L;
    s.lrow0[0] = o0;
    return s;
  }
  const int nch = 2 * p.cp_size;
  const int c0 = p.cp_rank, c1 = nch - 1 - p.cp_rank;
  s.n = 2;
  s.pos0[0] = chunk_lo(L, c0, nch);
  s.len[0] = chunk_lo(L, c0 + 1, nch) - s.pos0[0];
  s.pos0[1] = chunk_lo(L, c1, nch);
  s.len[1] = chunk_lo(L, c1 + 1, nch) - s.pos0[1];
  s.lrow0[0] = local0;
  s.lrow0[1] = local0 + s.len[0];
  return s;
}

__device__ __forceinline__ int local_len(const SchedParams& p, int b) {
  const int64_t L = p.offsets[b + 1] - p.offsets[b];
  if (p.targets_only) return candidates(p.num_targets, b, (int)L);
  if (p.cp_size == 1) return (int)L;
  const int nch = 2 * p.cp_size;
  const int c0 = p.cp_rank, c1 = nch - 1 - p.cp_rank;
  return (chunk_lo(L, c0 + 1, nch) - chunk_lo(L, c0, nch)) + (chunk_lo(L, c1 + 1, nch) - chunk_lo(L, c1, nch));
}

// Exclusive scan of one value per thread across the block; returns the
// thread's prefix and writes the block total to *total.  Wave-level inclusive
// scans with shuffles, then one pass over the 16 wave totals.
__device__ int64_t block_scan(int64_t v, int64_t* buf, int64_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int i = 0; i < kSchedThreads / 64; ++i) {
    const int64_t x = buf[i];
    before += i < wave ? x : 0;
    all += x;
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

// The same for the 64 lanes of one wave (no barrier): exclusive prefix, and
// the wave's total in every lane.
__device__ __forceinline__ int64_t wave_scan(int64_t v, int64_t* total) {
  const int lane = threadIdx.x & 63;
  int64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  *total = __shfl(incl, 63);
  return incl - v;
}

// Whether the stored score gradient can serve sequence b: its blocks cover
// 128-row query tiles at multiples of 128, so every query segment must start
// on such a boundary and end on one or at the sequence end (always so without
// context parallelism: one segment from 0 to L).
__device__ __forceinline__ bool g_aligned(const SchedParams& p, int b, int64_t local0) {
  const SegInfo s = seq_segments(p, b, local0);
  const int L = (int)(p.offsets[b + 1] - p.offsets[b]);
  bool ok = true;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    if (sg >= s.n) break;
    const int end = s.pos0[sg] + s.len[sg];
    ok = ok && s.pos0[sg] % kGRows == 0 && (end % kGRows == 0 || end == L);
  }
  return ok;
}

// Query tiles, key tiles and stored-G blocks of sequence b, whose rank-local
// rows start at local0.
struct SeqCounts {
  int64_t nq, nk, ng;
};

__device__ __forceinline__ SeqCounts seq_counts(const SchedParams& p, int b, int64_t local0) {
  SeqCounts c{0, 0, 0};
  const SegInfo s = seq_segments(p, b, local0);
  if (p.q_tile > 0)
#pragma unroll
    for (int sg = 0; sg < 2; ++sg)  // constant indices keep SegInfo in registers
      if (sg < s.n) c.nq += (s.len[sg] + p.q_tile - 1) / p.q_tile;
  const int64_t L = p.offsets[b + 1] - p.offsets[b];
  if (p.k_tile > 0) c.nk = (L + p.k_tile - 1) / p.k_tile;
  if (p.gblk_off) {  // stored-G blocks: n(n+1) per head, n = query tiles of kGRows rows
    const int64_t n = (L + kGRows - 1) / kGRows;
    c.ng = (int64_t)p.g_heads * n * (n + 1);
  }
  return c;
}

__device__ __forceinline__ int clampc(int64_t c, int hs) { return (int)(c < hs - 1 ? c : hs - 1); }

// Sequence owning flat tile j: the largest b with off[b] <= j.
__device__ __forceinline__ int owner(const int* off, int64_t B, int j) {
  int lo = 0, hi = (int)B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

struct QTile {
  int b, pos0, n;
  int64_t row0;
  int cost;  // key tiles the forward visits
};

// Key tiles of q_cost_tile keys visited by a query tile ending at position
// end (exclusive) that starts at pos0, with hist history rows: the causal
// prefix, but past the history only the tiles that hold the tile's own rows
// (a candidate sees no other candidate).
__device__ __forceinline__ int q_tile_cost(int pos0, int end, int hist, int ct) {
  const int ht = (min(end, hist) + ct - 1) / ct;
  if (end <= hist) return ht;
  const int d0 = max(max(pos0, hist) / ct, ht), last = (end - 1) / ct;
  return ht + (last >= d0 ? last - d0 + 1 : 0);
}

// Flat query tile j: tiles of q_tile rows over the sequence's segments.
__device__ __forceinline__ QTile query_tile(const SchedParams& p, int j) {
  const int b = owner(p.qtile_off, p.B, j);
  const SegInfo s = seq_segments(p, b, p.local_off[b]);
  int i = j - p.qtile_off[b];
  const int n0 = (s.len[0] + p.q_tile - 1) / p.q_tile;
  const int sg = i < n0 ? 0 : 1;
  if (sg == 1) i -= n0;
  const int r = i * p.q_tile;
  // selects rather than an indexed read keep SegInfo in registers
  const int pos0 = (sg ? s.pos0[1] : s.pos0[0]) + r, n = min(p.q_tile, (sg ? s.len[1] : s.len[0]) - r);
  const int L = (int)(p.offsets[b + 1] - p.offsets[b]);
  const int hist = L - candidates(p.num_targets, b, L);
  return QTile{b, pos0, n, (sg ? s.lrow0[1] : s.lrow0[0]) + r, q_tile_cost(pos0, pos0 + n, hist, p.q_cost_tile)};
}

struct KTile {
  int b, k0, n;
  int64_t cost;
};

// Flat key tile j: k_tile keys from k0; cost = query steps at or after k0.
__device__ __forceinline__ KTile key_tile(const SchedParams& p, int j) {
  const int b = owner(p.ktile_off, p.B, j);
  const int L = (int)(p.offsets[b + 1] - p.offsets[b]);
  const int k0 = (j - p.ktile_off[b]) * p.k_tile;
  const SegInfo s = seq_segments(p, b, p.local_off[b]);
  int64_t cost = 0;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {  // constant indices keep SegInfo in registers
    if (sg >= s.n) break;
    const int from = max(s.pos0[sg], k0), to = s.pos0[sg] + s.len[sg];
    if (to > from) cost += (to - from + p.k_cost_tile - 1) / p.k_cost_tile;
  }
  return KTile{b, k0, min(p.k_tile, L - k0), cost};
}

// #{k in [1, nb) : E_k <= m}
__device__ int bucket_search(uint64_t m, const EdgeArg& edges, int nb) {
  int lo = 0, hi = nb - 1;  // answer in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((uint64_t)edges.e[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Entry idx = (z << 5) | j of the exact-bucket table: the integers m whose
// leading-zero count is z and whose five bits after the leading one are j.
// With b0 the bucket of the smallest such m, the entry is {E, b0} when an edge
// E lies above it within the sub-bin, else {0, b0 - 1} (the compare always
// adds one).  At most one edge lies in a sub-bin for NB <= 512 (checked on
// the host).  Index patterns no integer produces hold {0, 0xFFFFFFFF}.
__device__ u32x2 lut_entry(int idx, const EdgeArg& edges, int nb) {
  const int e = 31 - (idx >> 5), j = idx & 31;
  uint64_t lo, hi;
  if (e >= 5) {
    lo = (uint64_t)(32 + j) << (e - 5);
    hi = lo + (1ull << (e - 5)) - 1;
  } else {
    const int step = 1 << (5 - e);
    if (j % step) return u32x2{0u, 0xFFFFFFFFu};
    lo = hi = (1ull << e) + (uint64_t)(j / step);
  }
  const int b0 = bucket_search(lo, edges, nb);
  if (b0 + 1 < nb && (uint64_t)edges.e[b0 + 1] <= hi) return u32x2{edges.e[b0 + 1], (uint32_t)b0};
  return u32x2{0u, (uint32_t)(b0 - 1)};
}

// Parts of a query tile whose walk covers `cost` key tiles, at most `cap` key
// tiles per part; part k covers walk positions [k cost / n, (k+1) cost / n).
__device__ __forceinline__ int nparts(int cost, int cap) { return cost > cap ? (cost + cap - 1) / cap : 1; }
__device__ __forceinline__ int part_begin(int cost, int n, int k) { return (int)((int64_t)k * cost / n); }

// Query tiles cached in LDS while splitting (the split is only considered
// below 2 kQuerySlots (tile, head) items, so at most this many tiles).
constexpr int kSplitTileCache = 2 * kQuerySlots;
static_assert(kSplitTileCache <= kSchedThreads, "one pass over the cached tiles");

}  // namespace

__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const SchedParams p, const EdgeArg edges) {
  __shared__ int histq[kSchedHist];
  __shared__ int histk[kSchedHist];
  __shared__ int64_t scan[kSchedThreads];
  __shared__ QTile qcache[kSplitTileCache];
  __shared__ int qslot[kSplitTileCache];
  __shared__ int qcost_max;
  __shared__ int g_ok;
  const int t = threadIdx.x;
  const int hs = p.hist_size;

  for (int i = t; i <= p.NB; i += kSchedThreads) p.edges_out[i] = edges.e[i];
  for (int i = t; i < kLutSize; i += kSchedThreads) p.lut_out[i] = lut_entry(i, edges, p.NB);
  if (p.dw)
    for (int i = t; i < p.dw_count; i += kSchedThreads) p.dw[i] = 0.0f;
  for (int i = t; i < hs; i += kSchedThreads) {
    histq[i] = 0;
    histk[i] = 0;
  }
  if (t == 0) {
    qcost_max = 0;
    g_ok = 1;
  }

  // Rank-local offsets, then tile counts per sequence, scanned: sequence b
  // owns query tiles [qtile_off[b], qtile_off[b+1]) and key tiles
  // [ktile_off[b], ktile_off[b+1]) of the flat tile order, so that the passes
  // below run one thread per tile.  Key tiles and stored-G blocks share one
  // scan: both totals stay below 2^31 (the stored-G path is only taken for at
  // most 2^20 blocks).  Up to 64 sequences, one wave does all of it.
  int64_t qcarry = 0, kcarry = 0, gcarry = 0;
  if (p.B <= 64) {
    if (t < 64) {
      const int b = t;
      const bool in = b < p.B;
      int64_t tot;
      const int64_t pre = wave_scan(in ? local_len(p, b) : 0, &tot);
      if (in) p.local_off[b] = pre;
      if (t == 0) p.local_off[p.B] = tot;
      const SeqCounts c = in ? seq_counts(p, b, pre) : SeqCounts{0, 0, 0};
      if (p.gblk_off && in && !g_aligned(p, b, pre)) g_ok = 0;
      int64_t qtot, kgtot;
      const int64_t qpre = wave_scan(c.nq, &qtot);
      const int64_t kgpre = wave_scan(c.nk | (c.ng << 32), &kgtot);
      if (in) {
        p.qtile_off[b] = (int)qpre;
        p.ktile_off[b] = (int)(kgpre & 0xFFFFFFFF);
        if (p.gblk_off) p.gblk_off[b] = kgpre >> 32;
      }
      if (t == 0) {
        scan[0] = qtot;
        scan[1] = kgtot;
      }
    }
    __syncthreads();
    qcarry = scan[0];
    kcarry = scan[1] & 0xFFFFFFFF;
    gcarry = scan[1] >> 32;
  } else {
    int64_t carry = 0;
    for (int64_t base = 0; base < p.B; base += kSchedThreads) {
      const int64_t b = base + t;
      const int64_t len = b < p.B ? local_len(p, (int)b) : 0;
      int64_t tot;
      const int64_t pre = block_scan(len, scan, &tot);
      if (b < p.B) p.local_off[b] = carry + pre;
      carry += tot;
    }
    if (t == 0) p.local_off[p.B] = carry;
    __syncthreads();
    for (int64_t base = 0; base < p.B; base += kSchedThreads) {
      const int64_t b = base + t;
      const SeqCounts c = b < p.B ? seq_counts(p, (int)b, p.local_off[b]) : SeqCounts{0, 0, 0};
      // (read by thread 0 after the barriers of the scans below)
      if (p.gblk_off && b < p.B && !g_aligned(p, (int)b, p.local_off[b])) g_ok = 0;
      int64_t qtot, kgtot;
      const int64_t qpre = block_scan(c.nq, scan, &qtot);
      const int64_t kgpre = block_scan(c.nk | (c.ng << 32), scan, &kgtot);
      if (b < p.B) {
        p.qtile_off[b] = (int)(qcarry + qpre);
        p.ktile_off[b] = (int)(kcarry + (kgpre & 0xFFFFFFFF));
        if (p.gblk_off) p.gblk_off[b] = gcarry + (kgpre >> 32);
      }
      qcarry += qtot;
      kcarry += kgtot & 0xFFFFFFFF;
      gcarry += kgtot >> 32;
    }
  }
  if (t == 0) {
    p.qtile_off[p.B] = (int)qcarry;
    p.ktile_off[p.B] = (int)kcarry;
    if (p.gblk_off) p.gblk_off[p.B] = gcarry;
    p.ctr[kCtrGMode] = p.gblk_off ? g_ok : 0;
  }
  __syncthreads();
  const int nqt = (int)qcarry, nkt = (int)kcarry;

  // Key-range splitting of long query tiles, considered only when the (tile,
  // head) items cannot fill 2 kQuerySlots workgroups, and done only when the
  // longest tile exceeds 1.5 times both the mean load of a workgroup slot and
  // kMinPartTiles (else the longest-first schedule is balanced already):
  // then at most cap = max(kMinPartTiles, ceil(total cost x heads /
  // (3 kQuerySlots))) key tiles per part, about three items per workgroup.
  // The host sized the item list and the partial slots for q_extra parts
  // beyond one per tile (a bound the cap keeps); the cap doubles should it not.
  const bool split = p.q_extra > 0 && nqt > 0 && (int64_t)nqt * p.heads < 2 * kQuerySlots;
  int cap = 0x3FFFFFFF;
  if (split) {
    const int j = t;  // nqt <= kSplitTileCache <= kSchedThreads: one tile per thread
    int64_t csum = 0;
    if (j < nqt) {
      qcache[j] = query_tile(p, j);
      csum = qcache[j].cost;
      atomicMax(&qcost_max, qcache[j].cost);
    }
    int64_t tot;
    block_scan(csum, scan, &tot);  // its barriers also publish qcost_max
    const int64_t mean = (tot * p.heads + kQuerySlots - 1) / kQuerySlots;
    if (2 * (int64_t)qcost_max > 3 * max<int64_t>(mean, kMinPartTiles))
      cap = (int)max<int64_t>(kMinPartTiles, (tot * p.heads + 3 * kQuerySlots - 1) / (3 * kQuerySlots));
    // partial slots (low half) and split-list index (high half) of each split
    // tile; the extra parts are the slots less the split tiles
    int np;
    int64_t pre, stot;
    for (;;) {
      np = j < nqt ? nparts(qcache[j].cost, cap) : 1;
      pre = block_scan(np > 1 ? ((int64_t)1 << 32) | np : 0, scan, &stot);
      if ((stot & 0xFFFFFFFF) - (stot >> 32) <= p.q_extra) break;
      cap *= 2;
    }
    if (j < nqt) {
      qslot[j] = np > 1 ? (int)(pre & 0xFFFFFFFF) : -1;
      if (np > 1) p.splits[pre >> 32] = SplitTile{(int)qcache[j].row0, qcache[j].n, (int)(pre & 0xFFFFFFFF), np};
    }
    if (t == 0) p.ctr[kCtrSplits] = (int)(stot >> 32);
    __syncthreads();
  } else if (t == 0) {
    p.ctr[kCtrSplits] = 0;
  }

  // Pass 1: cost histograms (of the parts when splitting).
  for (int j = t; j < nqt; j += kSchedThreads) {
    if (split) {
      const int c = qcache[j].cost, np = nparts(c, cap);
      for (int k = 0; k < np; ++k) atomicAdd(&histq[clampc(part_begin(c, np, k + 1) - part_begin(c, np, k), hs)], 1);
    } else {
      atomicAdd(&histq[clampc(query_tile(p, j).cost, hs)], 1);
    }
  }
  for (int j = t; j < nkt; j += kSchedThreads) atomicAdd(&histk[clampc(key_tile(p, j).cost, hs)], 1);
  __syncthreads();

  // Descending exclusive scans of both histograms at once (query counts in
  // the low half, key counts in the high half; both totals stay below 2^31):
  // start[c] = number of tiles with cost > c.  Each thread rewrites only the
  // bin it read.  Up to 64 bins, one wave scans them.
  int64_t carry2 = 0;
  if (hs <= 64) {
    if (t < 64) {
      const int c = hs - 1 - t;
      const int64_t v = c >= 0 ? ((int64_t)histk[c] << 32) | (uint32_t)histq[c] : 0;
      const int64_t pre = wave_scan(v, &carry2);
      if (c >= 0) {
        histq[c] = (int)(pre & 0xFFFFFFFF);
        histk[c] = (int)(pre >> 32);
      }
    }
  } else {
    for (int base = 0; base < hs; base += kSchedThreads) {
      const int c = hs - 1 - (base + t);
      const int64_t v = c >= 0 ? ((int64_t)histk[c] << 32) | (uint32_t)histq[c] : 0;
      int64_t tot;
      const int64_t pre = carry2 + block_scan(v, scan, &tot);
      if (c >= 0) {
        histq[c] = (int)(pre & 0xFFFFFFFF);
        histk[c] = (int)(pre >> 32);
      }
      carry2 += tot;
    }
  }
  if (t == 0) {
    p.ctr[kCtrQTiles] = (int)(carry2 & 0xFFFFFFFF);
    p.ctr[kCtrKTiles] = (int)(carry2 >> 32);
  }
  __syncthreads();

  // Pass 2: scatter.
  for (int j = t; j < nqt; j += kSchedThreads) {
    const QTile q = split ? qcache[j] : query_tile(p, j);
    const int np = split ? nparts(q.cost, cap) : 1;
    for (int k = 0; k < np; ++k) {
      const int w0 = part_begin(q.cost, np, k), w1 = part_begin(q.cost, np, k + 1);
      const int slot = atomicAdd(&histq[clampc(w1 - w0, hs)], 1);
      p.qitems[slot] = Item{q.b, (int)q.row0, q.pos0, q.n, w0, w1, np > 1 ? qslot[j] + k : -1, 0};
    }
  }
  for (int j = t; j < nkt; j += kSchedThreads) {
    const KTile k = key_tile(p, j);
    const int slot = atomicAdd(&histk[clampc(k.cost, hs)], 1);
    p.kitems[slot] = Item{k.b, (int)(p.offsets[k.b] + k.k0), k.k0, k.n, 0, 0, -1, 0};
  }
  if (t == 0) {
    p.ctr[kCtrQNext] = 0;
    p.ctr[kCtrKNext] = 0;
    p.ctr[kCtrQNext2] = 0;
  }
}

hipError_t launch_sched(const SchedParams& p, const EdgeArg& edges, hipStream_t s) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kSchedThreads), 0, s, p, edges);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Check of the offsets contract (run only when the caller asks for it): the
// jagged layout of §2.2 of the CP paper (values plus offsets plus max_lengths)
// is valid when offsets start at 0, never decrease and end at the row count,
// and no sequence is longer than the stated maximum.  One workgroup; each
// thread folds its sequences into a bit set and two sums, which thread 0
// combines.
// ---------------------------------------------------------------------------
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_kernel(const CheckParams p, int* flag) {
  __shared__ int bits;
  __shared__ unsigned __int128 sq[kCheckThreads];
  __shared__ unsigned long long rows[kCheckThreads];
  const int t = threadIdx.x;
  if (t == 0) bits = 0;
  __syncthreads();
  int mine = 0;
  unsigned __int128 sumsq = 0;
  unsigned long long nrows = 0;
  for (int64_t b = t; b < p.B; b += kCheckThreads) {
    const int64_t lo = p.offsets[b], hi = p.offsets[b + 1];
    if (hi < lo) {
      mine |= kBadOrder;
      continue;
    }
    const int64_t L = hi - lo;
    if (L > p.max_seq_len) mine |= kBadMaxLen;
    sumsq += (unsigned __int128)L * (unsigned __int128)L;
    if (p.total_q >= 0) {
      if (p.targets_only) {
        const int64_t m = p.num_targets ? p.num_targets[b] : 0;
        nrows += (unsigned long long)(m < 0 ? 0 : (m > L ? L : m));
      } else if (p.cp_size > 1) {
        const int64_t nch = 2 * (int64_t)p.cp_size;
        const int64_t c0 = p.cp_rank, c1 = nch - 1 - p.cp_rank;
        nrows += (unsigned long long)(((c0 + 1) * L / nch - c0 * L / nch) + ((c1 + 1) * L / nch - c1 * L / nch));
      } else {
        nrows += (unsigned long long)L;
      }
    }
  }
  if (t == 0) {
    if (p.offsets[0] != 0) mine |= kBadFirst;
    if (p.offsets[p.B] != p.total_kv) mine |= kBadTotal;
  }
  if (mine) atomicOr(&bits, mine);
  sq[t] = sumsq;
  rows[t] = nrows;
  __syncthreads();
  if (t == 0) {
    unsigned __int128 s2 = 0;
    unsigned long long r = 0;
    for (int i = 0; i < kCheckThreads; ++i) {
      s2 += sq[i];
      r += rows[i];
    }
    int out = bits;
    if (p.sum_sq_len > 0 && s2 > (unsigned __int128)p.sum_sq_len) out |= kBadSumSq;
    if (p.total_q >= 0 && r != (unsigned long long)p.total_q) out |= kBadRows;
    *flag = out;
  }
}

// The check's result on each device: a file-scope device variable, one copy
// per GPU, read back by the host after the check kernel.
__device__ int g_check_flag;

}  // namespace

hipError_t launch_check(const CheckParams& p, int* flag, hipStream_t s) {
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, s, p, flag);
  return hipGetLastError();
}

hipError_t check_flag_ptr(int** out) {
  static std::mutex mu;
  static int* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_check_flag));
    if (e != hipSuccess) return e;
    cache[dev] = static_cast<int*>(ptr);
  }
  *out = cache[dev];
  return hipSuccess;
}

}  // namespace hstu
