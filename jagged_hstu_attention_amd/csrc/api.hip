// Host side of the C ABI declared in include/hstu.h: argument validation,
// workspace layout, the integer bucket-edge table, and kernel launches on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "attn.h"
#include "bias.h"
#include "hstu.h"
#include "layer.h"
#include "sl.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HSTU_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Bucket edges E_k = ceil(2^(32k/NB)).  For 32k/NB integral the edge is an
// exact power of two.  Otherwise 2^(32k/NB) is irrational and the long-double
// value is accurate to ~2^-31 absolute; a candidate is accepted once a
// multi-word integer comparison confirms (E-1)^NB < 2^(32k) <= E^NB.
// ---------------------------------------------------------------------------
struct BigU {
  std::vector<uint32_t> w;  // little-endian words
  explicit BigU(uint64_t v = 0) {
    while (v) {
      w.push_back((uint32_t)v);
      v >>= 32;
    }
  }
  void mul(uint32_t m) {
    uint64_t carry = 0;
    for (auto& x : w) {
      const uint64_t t = (uint64_t)x * m + carry;
      x = (uint32_t)t;
      carry = t >> 32;
    }
    if (carry) w.push_back((uint32_t)carry);
  }
  // compare with 2^e: -1, 0, 1
  int cmp_pow2(int64_t e) const {
    size_t n = w.size();
    while (n && w[n - 1] == 0) --n;
    if (n == 0) return -1;
    const int64_t top = (int64_t)(n - 1) * 32 + (31 - __builtin_clz(w[n - 1]));
    if (top != e) return top < e ? -1 : 1;
    // leading bit matches: equal iff all lower bits are zero
    if (w[n - 1] & ~(1u << (top % 32))) return 1;
    for (size_t i = 0; i + 1 < n; ++i)
      if (w[i]) return 1;
    return 0;
  }
};

int cmp_pow_vs_pow2(uint64_t x, int64_t n, int64_t e) {  // sign of x^n - 2^e
  BigU v(1);
  for (int64_t i = 0; i < n; ++i) v.mul((uint32_t)x);
  return v.cmp_pow2(e);
}

bool edge_ok(uint64_t c, int64_t k, int64_t nb) {
  // c^nb >= 2^(32k) and (c-1)^nb < 2^(32k)
  return cmp_pow_vs_pow2(c, nb, 32 * k) >= 0 && (c == 0 || cmp_pow_vs_pow2(c - 1, nb, 32 * k) < 0);
}

void compute_edges(int64_t nb, uint32_t* e) {
  e[0] = 0;
  for (int64_t k = 1; k < nb; ++k) {
    const int64_t num = 32 * k;
    uint64_t c;
    if (num % nb == 0) {
      c = 1ull << (num / nb);
    } else {
      const long double y = std::exp2((long double)num / (long double)nb);
      c = (uint64_t)std::ceil(y);
      const long double frac_lo = y - std::floor(y);
      if (frac_lo < 1e-6L || frac_lo > 1.0L - 1e-6L) {
        // near an integer: settle exactly
        if (!edge_ok(c, k, nb)) c = edge_ok(c + 1, k, nb) ? c + 1 : c - 1;
      }
    }
    e[k] = (uint32_t)c;
  }
  e[nb] = 0xFFFFFFFFu;
}

// The kernels' exact-bucket table splits every octave [2^e, 2^(e+1)) into 32
// sub-bins and assumes no sub-bin holds two edges.  Check it for this table.
int64_t bucket_of_host(uint64_t m, const uint32_t* e, int64_t nb) {
  int64_t c = 0;
  for (int64_t k = 1; k < nb; ++k) c += m >= e[k] ? 1 : 0;
  return c;
}

bool subbins_hold_one_edge(const uint32_t* e, int64_t nb) {
  for (int oct = 5; oct < 32; ++oct)
    for (uint64_t j = 0; j < 32; ++j) {
      const uint64_t lo = (32 + j) << (oct - 5), hi = lo + (1ull << (oct - 5)) - 1;
      if (bucket_of_host(hi, e, nb) - bucket_of_host(lo, e, nb) > 1) return false;
    }
  return true;  // octaves below 5: a sub-bin holds at most one integer
}

struct EdgeCache {
  std::mutex mu;
  int64_t nb = -1;
  bool lut_ok = false;
  hstu::EdgeArg arg;
};
EdgeCache g_edges;

// Returns false when the exact-bucket table cannot represent these edges.
bool get_edges(int64_t nb, hstu::EdgeArg* out) {
  std::lock_guard<std::mutex> lk(g_edges.mu);
  if (g_edges.nb != nb) {
    std::memset(&g_edges.arg, 0, sizeof(g_edges.arg));
    compute_edges(nb, g_edges.arg.e);
    g_edges.lut_ok = subbins_hold_one_edge(g_edges.arg.e, nb);
    g_edges.nb = nb;
  }
  *out = g_edges.arg;
  return g_edges.lut_ok;
}

// Cached compute-unit count per device.
int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t ctr, edges, lut, dw_acc, local_off, tile_off, qitems, kitems, splits, parts, gblk_off, g, total;
  int64_t max_qtiles, max_ktiles, q_extra, g_blocks;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Key-range splitting of long query tiles (the scheduler decides it on the
// device): only possible when the (tile, head) items, at most max_qtiles x H,
// cannot fill 2 kQuerySlots workgroups.  The scheduler keeps the parts beyond
// one per tile within min(3 kQuerySlots / H, max_qtiles x ceil(max_seq_len /
// 64) / kMinPartTiles), a bound that sizes the item list (tiles plus extra
// parts), the split list (one entry per split tile, at most one per extra
// part) and the partial slots (a split tile has at least two parts: at most
// twice the extra parts), each slot [H][kSplitRows][d] fp32.
int64_t q_extra_for(const hstu_problem_t* p, int64_t max_qtiles) {
  if (max_qtiles * p->num_heads >= 2 * hstu::kQuerySlots) return 0;
  const int64_t tile_cost = cdiv(p->max_seq_len, hstu::attn_k_tile_keys());
  if (tile_cost <= hstu::kMinPartTiles) return 0;  // no walk is long enough to split
  return std::min<int64_t>(cdiv(3 * hstu::kQuerySlots, p->num_heads),
                           cdiv(max_qtiles * tile_cost, hstu::kMinPartTiles));
}

// Stored score gradients (backward, bf16, d >= 64): the dK/dV pass writes G,
// the dQ pass reads it instead of recomputing it (for a context-parallel
// share only when its chunk boundaries fall on 128-row boundaries, which the
// scheduler checks on the device; the blocks cover the whole sequences).  Blocks needed:
// sum over sequences and heads of n(n+1), n = ceil(L / kGRows).  Bound from
// host metadata (every L <= max_seq_len): n <= N = ceil(max_seq_len / kGRows)
// and sum n <= ceil(T / kGRows) + B, so H (N + 1) (ceil(T / kGRows) + B); when
// the caller states sum_sq_len (sum of L^2), also the bound below from it.
// 0 (recompute) when the path does not apply, the caller asks for the
// memory-efficient backward, or the bound passes kGMaxBytes.
constexpr int64_t kGMaxBytes = 16ll << 30;
int64_t g_blocks_for(const hstu_problem_t* p) {
  if (p->dtype != HSTU_BF16 || p->d_qk < 64 || p->total_kv == 0 || (p->flags & HSTU_FLAG_RECOMPUTE_BWD))
    return 0;
  const int64_t n = cdiv(p->max_seq_len, hstu::kGRows);
  int64_t per_head = (n + 1) * (cdiv(p->total_kv, hstu::kGRows) + p->num_seqs);
  if (p->sum_sq_len > 0) {
    // n_b (n_b + 1) <= (L_b + 127)(L_b + 255) / 128^2 for n_b = ceil(L_b / 128),
    // summed: (sum L^2 + 382 T + 32385 B) / 16384
    const int64_t r = hstu::kGRows;
    const int64_t sq = std::min(p->sum_sq_len, p->max_seq_len * p->total_kv);  // sum L^2 <= max L * sum L
    const int64_t tight = cdiv(sq + (3 * r - 2) * p->total_kv + (r - 1) * (2 * r - 1) * p->num_seqs, r * r);
    per_head = std::min(per_head, tight);
  }
  const int64_t blocks = p->num_heads * per_head;
  return blocks > kGMaxBytes / hstu::kGBlockBytes ? 0 : blocks;
}

Layout layout_for(const hstu_problem_t* p, bool backward, bool allow_split = true) {
  // a forward whose schedule the backward shares builds the backward's lists too
  backward = backward || (p->flags & HSTU_FLAG_SHARED_SCHEDULE);
  Layout l{};
  const int64_t segs = p->cp_size == 1 ? 1 : 2;
  l.max_qtiles = cdiv(p->total_q, hstu::attn_q_tile_rows()) + segs * p->num_seqs;
  l.max_ktiles = backward ? cdiv(p->total_kv, hstu::attn_bwd_key_tile(p->dtype == HSTU_BF16, (int)p->d_qk)) + p->num_seqs : 0;
  size_t off = 0;
  l.ctr = off;
  off = align_up(off + hstu::kCtrCount * sizeof(int));
  l.edges = off;
  off = align_up(off + (hstu::kMaxBuckets + 4) * sizeof(uint32_t));
  l.lut = off;
  off = align_up(off + hstu::kLutSize * sizeof(hstu::u32x2));
  l.dw_acc = off;
  off = align_up(off + (size_t)p->num_heads * p->num_buckets * sizeof(float));
  l.local_off = off;
  off = align_up(off + (size_t)(p->num_seqs + 1) * sizeof(int64_t));
  l.tile_off = off;
  off = align_up(off + (size_t)2 * (p->num_seqs + 1) * sizeof(int));
  l.q_extra = allow_split ? q_extra_for(p, l.max_qtiles) : 0;
  l.qitems = off;
  off = align_up(off + (size_t)(l.max_qtiles + l.q_extra) * sizeof(hstu::Item));
  l.kitems = off;
  off = align_up(off + (size_t)l.max_ktiles * sizeof(hstu::Item));
  l.splits = off;
  off = align_up(off + (size_t)l.q_extra * sizeof(hstu::SplitTile));
  l.parts = off;
  off = align_up(off + (size_t)(2 * l.q_extra * p->num_heads) * hstu::kSplitRows * p->d_v * sizeof(float));
  l.g_blocks = backward ? g_blocks_for(p) : 0;
  l.gblk_off = off;
  off = align_up(off + (l.g_blocks ? (size_t)(p->num_seqs + 1) * sizeof(int64_t) : 0));
  l.g = off;
  off = align_up(off + (size_t)l.g_blocks * hstu::kGBlockBytes);
  l.total = off;
  return l;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// q_subset: the query rows may be a subset of the key rows with cp_size 1
// (the candidates-only forward).
int validate(const hstu_problem_t* p, bool q_subset = false) {
  if (!p) return fail(HSTU_EINVAL, "problem is NULL");
  if (p->dtype != HSTU_BF16 && p->dtype != HSTU_FP32) return fail(HSTU_EINVAL, "dtype %d is not bf16 (0) or fp32 (1)", p->dtype);
  if (p->flags & ~(HSTU_FLAG_RECOMPUTE_BWD | HSTU_FLAG_SHARED_SCHEDULE))
    return fail(HSTU_EINVAL, "unknown flags 0x%x", (unsigned)p->flags);
  if (p->sum_sq_len < 0) return fail(HSTU_EINVAL, "sum_sq_len %lld < 0", (long long)p->sum_sq_len);
  if (p->num_seqs < 0) return fail(HSTU_EINVAL, "num_seqs %lld < 0", (long long)p->num_seqs);
  if (p->num_heads < 1) return fail(HSTU_EINVAL, "num_heads %lld < 1", (long long)p->num_heads);
  if (p->d_qk != 32 && p->d_qk != 64 && p->d_qk != 128)
    return fail(HSTU_EUNSUPPORTED, "d_qk %lld not in {32, 64, 128}", (long long)p->d_qk);
  if (p->d_v != p->d_qk) return fail(HSTU_EUNSUPPORTED, "d_v %lld != d_qk %lld", (long long)p->d_v, (long long)p->d_qk);
  if (p->num_buckets < 1) return fail(HSTU_EINVAL, "num_buckets %lld < 1", (long long)p->num_buckets);
  if (p->num_buckets > hstu::kMaxBuckets)
    return fail(HSTU_EUNSUPPORTED, "num_buckets %lld > %d", (long long)p->num_buckets, hstu::kMaxBuckets);
  if (p->cp_size < 1) return fail(HSTU_EINVAL, "cp_size %lld < 1", (long long)p->cp_size);
  if (p->cp_rank < 0 || p->cp_rank >= p->cp_size)
    return fail(HSTU_EINVAL, "cp_rank %lld not in [0, %lld)", (long long)p->cp_rank, (long long)p->cp_size);
  if (p->cp_size > 1024) return fail(HSTU_EUNSUPPORTED, "cp_size %lld > 1024", (long long)p->cp_size);
  if (p->total_kv < 0 || p->total_q < 0) return fail(HSTU_EINVAL, "negative row count");
  if (p->cp_size == 1 && !q_subset && p->total_q != p->total_kv)
    return fail(HSTU_EINVAL, "total_q %lld != total_kv %lld with cp_size 1", (long long)p->total_q, (long long)p->total_kv);
  if (p->total_q > p->total_kv) return fail(HSTU_EINVAL, "total_q > total_kv");
  if (p->max_seq_len < 0) return fail(HSTU_EINVAL, "max_seq_len %lld < 0", (long long)p->max_seq_len);
  if (p->max_seq_len > p->total_kv) return fail(HSTU_EINVAL, "max_seq_len %lld > total_kv %lld", (long long)p->max_seq_len, (long long)p->total_kv);
  if (p->total_kv > 0 && p->max_seq_len == 0) return fail(HSTU_EINVAL, "max_seq_len is 0 but total_kv > 0");
  if (p->total_kv >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "total_kv %lld >= 2^31", (long long)p->total_kv);
  if (p->num_seqs >= (1ll << 30)) return fail(HSTU_EUNSUPPORTED, "num_seqs too large");
  if (p->num_heads * p->d_qk >= (1ll << 24)) return fail(HSTU_EUNSUPPORTED, "num_heads * d too large");
  const Layout l = layout_for(p, true);
  if ((l.max_qtiles + l.max_ktiles) * p->num_heads >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "too many work items");
  return HSTU_OK;
}

#define CHECK_PTR(ptr, name)                                                               \
  do {                                                                                     \
    if (!(ptr)) return fail(HSTU_EINVAL, "%s is NULL", name);                              \
    if (!aligned16(ptr)) return fail(HSTU_EINVAL, "%s is not 16-byte aligned", name);      \
  } while (0)

#define CHECK_PTR8(ptr, name)                                                              \
  do {                                                                                     \
    if (!(ptr)) return fail(HSTU_EINVAL, "%s is NULL", name);                              \
    if (((uintptr_t)(ptr) & 7) != 0) return fail(HSTU_EINVAL, "%s is not 8-byte aligned", name); \
  } while (0)

// ---------------------------------------------------------------------------
// Optional per-kernel timing (hstu_timing_*): events recorded on the launch
// stream around each launch; resolved when read.
// ---------------------------------------------------------------------------
struct TimingRec {
  int kernel;
  hipEvent_t start, stop;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimingRec> pending;
  double ms[HSTU_KERNEL_COUNT] = {};
  int64_t launches[HSTU_KERNEL_COUNT] = {};
};
Timing g_timing;

template <class F>
hipError_t timed(int kernel, hipStream_t s, F&& launch) {
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.on) return launch();
  }
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return launch();
  hipEventRecord(a, s);
  const hipError_t e = launch();
  hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.pending.push_back(TimingRec{kernel, a, b});
  return e;
}

void timing_resolve_locked() {
  for (auto& r : g_timing.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      g_timing.ms[r.kernel] += ms;
      g_timing.launches[r.kernel] += 1;
    }
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  g_timing.pending.clear();
}


int schedule(const hstu_problem_t* p, const Layout& l, const int64_t* offsets, char* ws, float* dw,
             hipStream_t s, bool backward, const int64_t* num_targets = nullptr, int targets_only = 0) {
  hstu::SchedParams sp{};
  sp.offsets = offsets;
  sp.num_targets = num_targets;
  sp.targets_only = targets_only;
  sp.B = p->num_seqs;
  sp.cp_size = (int)p->cp_size;
  sp.cp_rank = (int)p->cp_rank;
  sp.q_tile = hstu::attn_q_tile_rows();
  sp.q_cost_tile = hstu::attn_k_tile_keys();
  sp.k_tile = backward ? hstu::attn_bwd_key_tile(p->dtype == HSTU_BF16, (int)p->d_qk) : 0;
  sp.k_cost_tile = hstu::attn_bwd_q_step();
  // costs are at most ceil(max_seq_len / 64) + 2 tiles
  const int64_t max_cost = cdiv(p->max_seq_len, std::min(hstu::attn_k_tile_keys(), hstu::attn_bwd_q_step())) + 3;
  sp.hist_size = (int)std::min<int64_t>(hstu::kSchedHist, std::max<int64_t>(max_cost, 1));
  sp.local_off = reinterpret_cast<int64_t*>(ws + l.local_off);
  sp.qtile_off = reinterpret_cast<int*>(ws + l.tile_off);
  sp.ktile_off = sp.qtile_off + (p->num_seqs + 1);
  sp.qitems = reinterpret_cast<hstu::Item*>(ws + l.qitems);
  sp.kitems = reinterpret_cast<hstu::Item*>(ws + l.kitems);
  sp.ctr = reinterpret_cast<int*>(ws + l.ctr);
  sp.edges_out = reinterpret_cast<uint32_t*>(ws + l.edges);
  sp.lut_out = reinterpret_cast<hstu::u32x2*>(ws + l.lut);
  // the d(ts_weights) sums start at zero (dw: an explicit target instead, for
  // problems with nothing to attend)
  sp.dw = dw ? dw : reinterpret_cast<float*>(ws + l.dw_acc);
  sp.dw_count = (int)(p->num_heads * p->num_buckets);
  sp.gblk_off = backward && l.g_blocks ? reinterpret_cast<int64_t*>(ws + l.gblk_off) : nullptr;
  sp.g_heads = (int)p->num_heads;
  sp.heads = (int)p->num_heads;
  sp.q_extra = (int)l.q_extra;
  sp.splits = reinterpret_cast<hstu::SplitTile*>(ws + l.splits);
  sp.NB = (int)p->num_buckets;
  hstu::EdgeArg edges;
  if (!get_edges(p->num_buckets, &edges))
    return fail(HSTU_EUNSUPPORTED, "bucket table for num_buckets %lld has two edges in one sub-bin",
                (long long)p->num_buckets);
  const hipError_t e = timed(HSTU_KERNEL_SCHED, s, [&] { return hstu::launch_sched(sp, edges, s); });
  if (e != hipSuccess) return hip_fail(e, "scheduler launch");
  return HSTU_OK;
}

hstu::AttnParams attn_params(const hstu_problem_t* p, const Layout& l, char* ws) {
  hstu::AttnParams a{};
  a.local_off = reinterpret_cast<const int64_t*>(ws + l.local_off);
  a.qitems = reinterpret_cast<const hstu::Item*>(ws + l.qitems);
  a.kitems = reinterpret_cast<const hstu::Item*>(ws + l.kitems);
  a.ctr = reinterpret_cast<int*>(ws + l.ctr);
  a.edges = reinterpret_cast<const uint32_t*>(ws + l.edges);
  a.lut = reinterpret_cast<const hstu::u32x2*>(ws + l.lut);
  a.dw_acc = reinterpret_cast<float*>(ws + l.dw_acc);
  if (l.q_extra) {
    a.parts = reinterpret_cast<float*>(ws + l.parts);
    a.splits = reinterpret_cast<const hstu::SplitTile*>(ws + l.splits);
  }
  if (l.g_blocks) {
    a.g = reinterpret_cast<uint16_t*>(ws + l.g);
    a.gblk_off = reinterpret_cast<const int64_t*>(ws + l.gblk_off);
    a.g_blocks = l.g_blocks;
  }
  a.H = (int)p->num_heads;
  a.NB = (int)p->num_buckets;
  a.cp_size = (int)p->cp_size;
  a.cp_rank = (int)p->cp_rank;
  a.alpha = (float)(1.0 / std::sqrt((double)p->d_qk));
  return a;
}


// Optional device check of the offsets contract: with HSTU_VALIDATE set to a
// value other than "0" in the environment, every call first checks offsets
// (and the host metadata stated with them) on the device and waits for the
// result (one host synchronisation), returning HSTU_EINVAL before any other
// launch when the contract is broken.
bool validate_enabled() {
  const char* v = std::getenv("HSTU_VALIDATE");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

// Host-side call logging: with HSTU_LOG set to a value other than "0" in the
// environment, every entry point that launches or validates work writes one
// line to stderr: its name, the problem's sizes when it takes one, and the
// status it returns (with the error message when it is not HSTU_OK).
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("HSTU_LOG");
    return v && v[0] && std::strcmp(v, "0") != 0;
  }();
  return on;
}

int logged(const char* name, const hstu_problem_t* p, int rc) {
  if (!log_enabled()) return rc;
  static const char* const kStatus[] = {"HSTU_OK", "HSTU_EINVAL", "HSTU_EUNSUPPORTED", "HSTU_EWORKSPACE", "HSTU_EHIP"};
  const char* st = rc >= 0 && rc <= 4 ? kStatus[rc] : "?";
  if (p)
    std::fprintf(stderr,
                 "hstu: %s dtype=%d flags=%d B=%lld H=%lld d_qk=%lld d_v=%lld NB=%lld max_len=%lld T_kv=%lld "
                 "T_q=%lld cp=%lld/%lld -> %s%s%s\n",
                 name, (int)p->dtype, (int)p->flags, (long long)p->num_seqs, (long long)p->num_heads,
                 (long long)p->d_qk, (long long)p->d_v, (long long)p->num_buckets, (long long)p->max_seq_len,
                 (long long)p->total_kv, (long long)p->total_q, (long long)p->cp_rank, (long long)p->cp_size, st,
                 rc ? ": " : "", rc ? g_last_error.c_str() : "");
  else
    std::fprintf(stderr, "hstu: %s -> %s%s%s\n", name, st, rc ? ": " : "", rc ? g_last_error.c_str() : "");
  return rc;
}

int check_offsets(const hstu::CheckParams& cp, hipStream_t s) {
  if (!validate_enabled()) return HSTU_OK;
  static std::mutex mu;  // one flag per device: checks on one device take turns
  std::lock_guard<std::mutex> lk(mu);
  int* flag = nullptr;
  hipError_t e = hstu::check_flag_ptr(&flag);
  if (e != hipSuccess) return hip_fail(e, "offsets check flag");
  e = hstu::launch_check(cp, flag, s);
  if (e != hipSuccess) return hip_fail(e, "offsets check launch");
  int bits = 0;
  e = hipMemcpyAsync(&bits, flag, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "offsets check read-back");
  if (!bits) return HSTU_OK;
  std::string why;
  const struct { int bit; const char* text; } msgs[] = {
      {hstu::kBadFirst, "offsets[0] != 0"},
      {hstu::kBadOrder, "offsets decrease"},
      {hstu::kBadTotal, "offsets[B] != the row count"},
      {hstu::kBadMaxLen, "a sequence is longer than max_seq_len"},
      {hstu::kBadSumSq, "the sum of squared lengths exceeds sum_sq_len"},
      {hstu::kBadRows, "the query row count differs from what the offsets imply"}};
  for (const auto& m : msgs)
    if (bits & m.bit) why += (why.empty() ? "" : "; ") + std::string(m.text);
  return fail(HSTU_EINVAL, "offsets check (HSTU_VALIDATE): %s", why.c_str());
}

hstu::CheckParams check_params(const hstu_problem_t* p, const int64_t* offsets) {
  hstu::CheckParams c{};
  c.offsets = offsets;
  c.B = p->num_seqs;
  c.total_kv = p->total_kv;
  c.max_seq_len = p->max_seq_len;
  c.sum_sq_len = p->sum_sq_len;
  c.total_q = p->total_q;
  c.cp_size = (int)p->cp_size;
  c.cp_rank = (int)p->cp_rank;
  return c;
}

}  // namespace

extern "C" {

int hstu_version(void) { return 100; }

int hstu_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return HSTU_OK;
}

int hstu_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  timing_resolve_locked();
  for (int i = 0; i < HSTU_KERNEL_COUNT; ++i) {
    g_timing.ms[i] = 0.0;
    g_timing.launches[i] = 0;
  }
  return HSTU_OK;
}

int hstu_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= HSTU_KERNEL_COUNT) return fail(HSTU_EINVAL, "kernel id %d out of range", kernel);
  if (!total_ms || !launches) return fail(HSTU_EINVAL, "output pointer is NULL");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  timing_resolve_locked();
  *total_ms = g_timing.ms[kernel];
  *launches = g_timing.launches[kernel];
  return HSTU_OK;
}

const char* hstu_last_error(void) { return g_last_error.c_str(); }

static int hstu_bucket_edges_body(int64_t num_buckets, uint32_t* edges_out) {
  if (!edges_out) return fail(HSTU_EINVAL, "edges_out is NULL");
  if (num_buckets < 1) return fail(HSTU_EINVAL, "num_buckets %lld < 1", (long long)num_buckets);
  if (num_buckets > hstu::kMaxBuckets)
    return fail(HSTU_EUNSUPPORTED, "num_buckets %lld > %d", (long long)num_buckets, hstu::kMaxBuckets);
  hstu::EdgeArg e;
  get_edges(num_buckets, &e);
  std::memcpy(edges_out, e.e, sizeof(uint32_t) * (num_buckets + 1));
  return HSTU_OK;
}

size_t hstu_workspace_size(const hstu_problem_t* p, int backward) {
  if (validate(p, backward == 0) != HSTU_OK) return 0;  // a forward may query a subset of rows
  return layout_for(p, backward != 0).total;
}

namespace {

int fwd_impl(const hstu_problem_t* p, const void* q, const void* k, const void* v, const int64_t* offsets,
             const int64_t* num_targets, int targets_only, const int64_t* timestamps, const void* ts_weights,
             void* out, void* workspace, size_t workspace_bytes, void* stream, bool allow_split = true) {
  if (p->total_q == 0 || p->num_seqs == 0) return HSTU_OK;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(out, "out");
  CHECK_PTR8(offsets, "offsets");
  CHECK_PTR8(timestamps, "timestamps");
  if (!ts_weights) return fail(HSTU_EINVAL, "ts_weights is NULL");
  const Layout l = layout_for(p, false, allow_split);  // the backward's layout with HSTU_FLAG_SHARED_SCHEDULE
  if (!workspace) return fail(HSTU_EWORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(HSTU_EINVAL, "workspace is not 16-byte aligned");
  if (workspace_bytes < l.total)
    return fail(HSTU_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, l.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hstu::CheckParams cp = check_params(p, offsets);
  cp.num_targets = num_targets;
  cp.targets_only = targets_only;
  int rc = check_offsets(cp, s);
  if (rc != HSTU_OK) return rc;
  // with a shared schedule the forward also builds the backward's key lists
  const bool shared = (p->flags & HSTU_FLAG_SHARED_SCHEDULE) != 0;
  rc = schedule(p, l, offsets, ws, nullptr, s, shared, num_targets, targets_only);
  if (rc != HSTU_OK) return rc;
  hstu::AttnParams a = attn_params(p, l, ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.offsets = offsets;
  a.ts = timestamps;
  a.w = ts_weights;
  a.out = out;
  a.num_targets = num_targets;
  a.targets_only = targets_only;
  const int max_items = (int)((l.max_qtiles + l.q_extra) * p->num_heads);
  const bool bf16 = p->dtype == HSTU_BF16;
  hipError_t e = timed(HSTU_KERNEL_FWD, s, [&] {
    return hstu::launch_attn(a, bf16, (int)p->d_qk, 0, max_items, cu_count(), s);
  });
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  if (l.q_extra) {
    e = timed(HSTU_KERNEL_REDUCE, s, [&] { return hstu::launch_reduce(a, bf16, (int)p->d_v, 0, (int)l.q_extra, s); });
    if (e != hipSuccess) return hip_fail(e, "split-sum launch");
  }
  return HSTU_OK;
}

}  // namespace

static int hstu_jagged_attn_fwd_body(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                         const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = validate(p);
  if (rc != HSTU_OK) return rc;
  return fwd_impl(p, q, k, v, offsets, nullptr, 0, timestamps, ts_weights, out, workspace, workspace_bytes, stream);
}

static int hstu_jagged_attn_fwd_targets_body(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                                 const int64_t* offsets, const int64_t* num_targets, int q_targets_only,
                                 const int64_t* timestamps, const void* ts_weights, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const int rc = validate(p, q_targets_only == 1);
  if (rc != HSTU_OK) return rc;
  if (p->cp_size != 1) return fail(HSTU_EUNSUPPORTED, "candidates with cp_size %lld > 1", (long long)p->cp_size);
  if (p->flags & HSTU_FLAG_SHARED_SCHEDULE)
    return fail(HSTU_EUNSUPPORTED, "a shared schedule is for a forward and backward pair; candidates have no backward");
  if (q_targets_only != 0 && q_targets_only != 1) return fail(HSTU_EINVAL, "q_targets_only %d is not 0 or 1", q_targets_only);
  if (!q_targets_only && p->total_q != p->total_kv)
    return fail(HSTU_EINVAL, "total_q %lld != total_kv %lld with q_targets_only 0", (long long)p->total_q,
                (long long)p->total_kv);
  if (p->total_q > p->total_kv)
    return fail(HSTU_EINVAL, "total_q %lld > total_kv %lld", (long long)p->total_q, (long long)p->total_kv);
  if (p->num_seqs > 0 && p->total_kv > 0) CHECK_PTR8(num_targets, "num_targets");
  return fwd_impl(p, q, k, v, offsets, num_targets, q_targets_only, timestamps, ts_weights, out, workspace,
                  workspace_bytes, stream);
}

static int hstu_jagged_attn_bwd_body(const hstu_problem_t* p, const void* dout, const void* q, const void* k, const void* v,
                         const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* dq,
                         void* dk, void* dv, float* d_ts_weights, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int rc = validate(p);
  if (rc != HSTU_OK) return rc;
  if (p->num_seqs == 0 || p->total_kv == 0) {
    // Nothing to attend: gradients of an empty problem.  d_ts_weights still
    // has to be written (zeros); the scheduler does it, with no lists.
    if (!d_ts_weights) return fail(HSTU_EINVAL, "d_ts_weights is NULL");
    if (((uintptr_t)d_ts_weights & 3) != 0) return fail(HSTU_EINVAL, "d_ts_weights is not 4-byte aligned");
    if (p->num_seqs > 0) CHECK_PTR8(offsets, "offsets");  // the scheduler reads offsets[0 .. B]
    const Layout l = layout_for(p, true);
    if (!workspace) return fail(HSTU_EWORKSPACE, "workspace is NULL");
    if (!aligned16(workspace)) return fail(HSTU_EINVAL, "workspace is not 16-byte aligned");
    if (workspace_bytes < l.total)
      return fail(HSTU_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, l.total);
    if (p->num_seqs == 0) return schedule(p, l, offsets, static_cast<char*>(workspace), d_ts_weights,
                                          static_cast<hipStream_t>(stream), true);
    rc = check_offsets(check_params(p, offsets), static_cast<hipStream_t>(stream));
    if (rc != HSTU_OK) return rc;
    return schedule(p, l, offsets, static_cast<char*>(workspace), d_ts_weights, static_cast<hipStream_t>(stream),
                    true);
  }
  if (p->total_q > 0) {
    CHECK_PTR(dout, "dout");
    CHECK_PTR(q, "q");
    CHECK_PTR(dq, "dq");
  }
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(dk, "dk");
  CHECK_PTR(dv, "dv");
  CHECK_PTR8(offsets, "offsets");
  CHECK_PTR8(timestamps, "timestamps");
  if (!ts_weights) return fail(HSTU_EINVAL, "ts_weights is NULL");
  if (!d_ts_weights) return fail(HSTU_EINVAL, "d_ts_weights is NULL");
  if (((uintptr_t)d_ts_weights & 3) != 0) return fail(HSTU_EINVAL, "d_ts_weights is not 4-byte aligned");
  const Layout l = layout_for(p, true);
  if (!workspace) return fail(HSTU_EWORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(HSTU_EINVAL, "workspace is not 16-byte aligned");
  if (workspace_bytes < l.total)
    return fail(HSTU_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, l.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  rc = check_offsets(check_params(p, offsets), s);
  if (rc != HSTU_OK) return rc;
  // with a shared schedule the forward of this step built the lists already
  // (and reset the d(ts_weights) sums)
  if (!(p->flags & HSTU_FLAG_SHARED_SCHEDULE)) {
    rc = schedule(p, l, offsets, ws, nullptr, s, true);
    if (rc != HSTU_OK) return rc;
  }
  hstu::AttnParams a = attn_params(p, l, ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.offsets = offsets;
  a.ts = timestamps;
  a.w = ts_weights;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = d_ts_weights;
  const bool bf16 = p->dtype == HSTU_BF16;
  hipError_t e = timed(HSTU_KERNEL_BWD_KV, s, [&] {
    return hstu::launch_attn(a, bf16, (int)p->d_qk, 1, (int)(l.max_ktiles * p->num_heads), cu_count(), s);
  });
  if (e != hipSuccess) return hip_fail(e, "dK/dV launch");
  {
    // the dQ pass also publishes d(ts_weights) (it runs with no items when
    // there are no query rows)
    e = timed(HSTU_KERNEL_BWD_Q, s, [&] {
      return hstu::launch_attn(a, bf16, (int)p->d_qk, 2, (int)((l.max_qtiles + l.q_extra) * p->num_heads),
                               cu_count(), s);
    });
    if (e != hipSuccess) return hip_fail(e, "dQ launch");
    if (l.q_extra && p->total_q > 0) {
      e = timed(HSTU_KERNEL_REDUCE, s, [&] { return hstu::launch_reduce(a, bf16, (int)p->d_qk, 2, (int)l.q_extra, s); });
      if (e != hipSuccess) return hip_fail(e, "split-sum launch");
    }
  }
  return HSTU_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without allocation (hstu_jagged_attn_fwd_noalloc): its workspace is
// `scratch`, a file-scope device array of kScratchBytes that every GPU the
// library runs on holds until the process ends.  In host code the array's
// name is only a stand-in for the symbol: the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress (that device
// current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = 16u << 20;
__device__ __align__(256) char scratch[kScratchBytes];

int scratch_ptr(char** out) {
  static std::mutex mu;
  static char* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no-allocation forward: current device");
  if (dev < 0 || dev >= 64) return fail(HSTU_EUNSUPPORTED, "device index %d >= 64", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "no-allocation forward: scratch address");
    cache[dev] = static_cast<char*>(ptr);
  }
  *out = cache[dev];
  return HSTU_OK;
}

}  // namespace

extern "C" {

size_t hstu_noalloc_scratch_bytes(void) { return kScratchBytes; }

static int hstu_jagged_attn_fwd_noalloc_body(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                                 const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* out,
                                 void* stream) {
  int rc = validate(p);
  if (rc != HSTU_OK) return rc;
  if (p->flags & HSTU_FLAG_SHARED_SCHEDULE)
    return fail(HSTU_EUNSUPPORTED, "the no-allocation forward does not share its schedule with a backward");
  // the work lists must fit the static scratch: with split key walks if their
  // partial sums fit too, else without (each query tile then walks its keys
  // in one item)
  bool split = true;
  size_t need = layout_for(p, false, true).total;
  if (need > kScratchBytes) {
    split = false;
    need = layout_for(p, false, false).total;
  }
  if (need > kScratchBytes)
    return fail(HSTU_EWORKSPACE, "problem needs %zu bytes of scratch; the no-allocation forward has %zu", need,
                kScratchBytes);
  if (p->total_q == 0 || p->num_seqs == 0) return HSTU_OK;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(out, "out");
  CHECK_PTR8(offsets, "offsets");
  CHECK_PTR8(timestamps, "timestamps");
  if (!ts_weights) return fail(HSTU_EINVAL, "ts_weights is NULL");
  char* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != HSTU_OK) return rc;
  return fwd_impl(p, q, k, v, offsets, nullptr, 0, timestamps, ts_weights, out, ws, kScratchBytes, stream, split);
}

static int hstu_sl_select_body(const int64_t* offsets, int64_t num_seqs, int64_t total_rows, int64_t max_seq_len, double alpha,
                   const float* seq_uniform, const uint32_t* token_keys, int64_t* out_offsets, int64_t* out_index,
                   void* stream) {
  if (num_seqs < 0) return fail(HSTU_EINVAL, "num_seqs %lld < 0", (long long)num_seqs);
  if (total_rows < 0) return fail(HSTU_EINVAL, "total_rows %lld < 0", (long long)total_rows);
  if (total_rows >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "total_rows %lld >= 2^31", (long long)total_rows);
  if (num_seqs >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "num_seqs too large");
  if (max_seq_len < 0 || max_seq_len > total_rows)
    return fail(HSTU_EINVAL, "max_seq_len %lld not in [0, total_rows]", (long long)max_seq_len);
  if (!(alpha > 0.0) || !(alpha < 64.0)) return fail(HSTU_EINVAL, "alpha %g not in (0, 64)", alpha);
  if (num_seqs == 0) return HSTU_OK;
  CHECK_PTR8(offsets, "offsets");
  CHECK_PTR8(out_offsets, "out_offsets");
  if (!seq_uniform || ((uintptr_t)seq_uniform & 3)) return fail(HSTU_EINVAL, "seq_uniform is NULL or misaligned");
  if (token_keys && ((uintptr_t)token_keys & 3)) return fail(HSTU_EINVAL, "token_keys is not 4-byte aligned");
  if (total_rows > 0) CHECK_PTR8(out_index, "out_index");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hstu::CheckParams cp{};
  cp.offsets = offsets;
  cp.B = num_seqs;
  cp.total_kv = total_rows;
  cp.max_seq_len = max_seq_len;
  cp.total_q = -1;
  const int rc = check_offsets(cp, s);
  if (rc != HSTU_OK) return rc;
  const hipError_t e = timed(HSTU_KERNEL_SL, s, [&] {
    return hstu::launch_sl_select(offsets, num_seqs, alpha, seq_uniform, token_keys, out_offsets, out_index, s);
  });
  if (e != hipSuccess) return hip_fail(e, "stochastic length launch");
  return HSTU_OK;
}

static int hstu_gather_rows_body(const void* in, void* out, int64_t row_bytes, const int64_t* index, const int64_t* count,
                     int64_t max_rows, void* stream) {
  if (row_bytes < 1) return fail(HSTU_EINVAL, "row_bytes %lld < 1", (long long)row_bytes);
  if (max_rows < 0) return fail(HSTU_EINVAL, "max_rows %lld < 0", (long long)max_rows);
  if (max_rows > 0 && row_bytes > (1ll << 40) / max_rows) return fail(HSTU_EUNSUPPORTED, "max_rows * row_bytes >= 2^40");
  if (max_rows == 0) return HSTU_OK;
  if (!in || !out) return fail(HSTU_EINVAL, "in/out is NULL");
  CHECK_PTR8(index, "index");
  CHECK_PTR8(count, "count");
  int vec = 16;
  while (vec > 1 && (row_bytes % vec || ((uintptr_t)in | (uintptr_t)out) % vec)) vec >>= 1;
  if (vec == 2) vec = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(HSTU_KERNEL_GATHER, s, [&] {
    return hstu::launch_gather_rows(in, out, row_bytes, index, count, max_rows, vec, cu_count(), s);
  });
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return HSTU_OK;
}

static int hstu_layer_projection_body(const void* x, const void* w, int64_t total_rows, int64_t d_model, int64_t num_heads,
                          int64_t d_qk, int64_t d_v, void* u, void* v, void* q, void* k, void* stream) {
  if (total_rows < 0) return fail(HSTU_EINVAL, "total_rows %lld < 0", (long long)total_rows);
  if (num_heads < 1 || d_qk < 1 || d_v < 1 || d_model < 1) return fail(HSTU_EINVAL, "sizes must be positive");
  const int64_t tc = hstu::proj_tile_cols(), tk = hstu::proj_tile_k();
  if (d_model % tk) return fail(HSTU_EUNSUPPORTED, "d_model %lld is not a multiple of %lld", (long long)d_model, (long long)tk);
  if ((num_heads * d_v) % tc || (num_heads * d_qk) % tc)
    return fail(HSTU_EUNSUPPORTED, "H * d_v and H * d_qk must be multiples of %lld", (long long)tc);
  if (num_heads * (2 * d_v + 2 * d_qk) >= (1ll << 24) || d_model >= (1ll << 24))
    return fail(HSTU_EUNSUPPORTED, "projection too wide");
  if (total_rows >= (1ll << 31) / 1) {
    if (total_rows * d_model >= (1ll << 40)) return fail(HSTU_EUNSUPPORTED, "total_rows * d_model too large");
  }
  if (total_rows == 0) return HSTU_OK;
  CHECK_PTR(x, "x");
  CHECK_PTR(w, "w");
  CHECK_PTR(u, "u");
  CHECK_PTR(v, "v");
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  if ((total_rows + hstu::proj_tile_rows() - 1) / hstu::proj_tile_rows() >= 65536 ||
      hstu::proj_workgroups(total_rows, num_heads * (2 * d_v + 2 * d_qk)) >= (1ll << 31))
    return fail(HSTU_EUNSUPPORTED, "total_rows %lld too large for the projection grid", (long long)total_rows);
  hstu::ProjParams pp{};
  pp.x = x;
  pp.w = w;
  pp.out[0] = u;
  pp.out[1] = v;
  pp.out[2] = q;
  pp.out[3] = k;
  pp.width[0] = pp.width[1] = (int)(num_heads * d_v);
  pp.width[2] = pp.width[3] = (int)(num_heads * d_qk);
  pp.T = total_rows;
  pp.Dm = d_model;
  pp.N = num_heads * (2 * d_v + 2 * d_qk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(HSTU_KERNEL_PROJ, s, [&] { return hstu::launch_proj(pp, s); });
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return HSTU_OK;
}

static int hstu_layer_norm_gate_body(const void* o, const void* u, void* y, int64_t total_rows, int64_t width, double eps,
                         void* stream) {
  if (total_rows < 0) return fail(HSTU_EINVAL, "total_rows %lld < 0", (long long)total_rows);
  if (width < 8 || width % 8) return fail(HSTU_EUNSUPPORTED, "width %lld is not a positive multiple of 8", (long long)width);
  if (width > hstu::norm_max_width())
    return fail(HSTU_EUNSUPPORTED, "width %lld > %d", (long long)width, hstu::norm_max_width());
  if (!(eps >= 0.0) || !(eps < 1.0)) return fail(HSTU_EINVAL, "eps %g not in [0, 1)", eps);
  if (total_rows >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "total_rows too large");
  if (total_rows == 0) return HSTU_OK;
  CHECK_PTR(o, "o");
  CHECK_PTR(u, "u");
  CHECK_PTR(y, "y");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed(HSTU_KERNEL_NORM_GATE, s, [&] {
    return hstu::launch_norm_gate(o, u, y, total_rows, (int)width, (float)eps, s);
  });
  if (e != hipSuccess) return hip_fail(e, "norm-gate launch");
  return HSTU_OK;
}

static int hstu_cp_reorder_body(const void* in, void* out, int64_t row_bytes, const int64_t* offsets, int64_t num_seqs,
                    int64_t total_rows, int64_t max_seq_len, int64_t cp_size, int inverse, int64_t* out_offsets,
                    void* stream) {
  if (num_seqs < 0) return fail(HSTU_EINVAL, "num_seqs %lld < 0", (long long)num_seqs);
  if (total_rows < 0) return fail(HSTU_EINVAL, "total_rows %lld < 0", (long long)total_rows);
  if (total_rows >= (1ll << 42)) return fail(HSTU_EUNSUPPORTED, "total_rows %lld >= 2^42", (long long)total_rows);
  if (row_bytes < 1) return fail(HSTU_EINVAL, "row_bytes %lld < 1", (long long)row_bytes);
  if (cp_size < 1) return fail(HSTU_EINVAL, "cp_size %lld < 1", (long long)cp_size);
  if (cp_size > 1024) return fail(HSTU_EUNSUPPORTED, "cp_size %lld > 1024", (long long)cp_size);
  if (max_seq_len < 0 || max_seq_len > total_rows)
    return fail(HSTU_EINVAL, "max_seq_len %lld not in [0, total_rows]", (long long)max_seq_len);
  if (total_rows > 0 && max_seq_len == 0) return fail(HSTU_EINVAL, "max_seq_len is 0 but total_rows > 0");
  if (num_seqs == 0) return HSTU_OK;
  if (cp_size * num_seqs >= (1ll << 31)) return fail(HSTU_EUNSUPPORTED, "cp_size * num_seqs too large");
  if (!in || !out) return fail(HSTU_EINVAL, "in/out is NULL");
  CHECK_PTR8(offsets, "offsets");
  if (out_offsets && ((uintptr_t)out_offsets & 7)) return fail(HSTU_EINVAL, "out_offsets is not 8-byte aligned");
  const char* ib = static_cast<const char*>(in);
  const char* ob = static_cast<const char*>(out);
  const int64_t bytes = total_rows * row_bytes;
  if (total_rows > 0 && ib < ob + bytes && ob < ib + bytes) return fail(HSTU_EINVAL, "in and out overlap");
  const int64_t nch = 2 * cp_size;
  const int64_t max_pair_bytes = 2 * ((max_seq_len + nch - 1) / nch) * row_bytes;
  if (max_pair_bytes / (64 * 1024) >= 65535) return fail(HSTU_EUNSUPPORTED, "sequence too long for the reorder grid");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hstu::CheckParams cp{};
  cp.offsets = offsets;
  cp.B = num_seqs;
  cp.total_kv = total_rows;
  cp.max_seq_len = max_seq_len;
  cp.total_q = -1;
  const int rc = check_offsets(cp, s);
  if (rc != HSTU_OK) return rc;
  const hipError_t e = timed(HSTU_KERNEL_REORDER, s, [&] {
    return hstu::launch_reorder(in, out, row_bytes, offsets, num_seqs, total_rows, max_seq_len, (int)cp_size,
                                inverse != 0, out_offsets, s);
  });
  if (e != hipSuccess) return hip_fail(e, "reorder launch");
  return HSTU_OK;
}

}  // extern "C"

// Exported entry points: each runs its body and, with HSTU_LOG set, logs the call.
int hstu_bucket_edges(int64_t num_buckets, uint32_t* edges_out) {
  return logged("hstu_bucket_edges", nullptr, hstu_bucket_edges_body(num_buckets, edges_out));
}

int hstu_jagged_attn_fwd(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                         const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return logged("hstu_jagged_attn_fwd", p, hstu_jagged_attn_fwd_body(p, q, k, v, offsets, timestamps, ts_weights, out, workspace, workspace_bytes, stream));
}

int hstu_jagged_attn_fwd_targets(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                                 const int64_t* offsets, const int64_t* num_targets, int q_targets_only,
                                 const int64_t* timestamps, const void* ts_weights, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return logged("hstu_jagged_attn_fwd_targets", p, hstu_jagged_attn_fwd_targets_body(p, q, k, v, offsets, num_targets, q_targets_only, timestamps, ts_weights, out, workspace, workspace_bytes, stream));
}

int hstu_jagged_attn_bwd(const hstu_problem_t* p, const void* dout, const void* q, const void* k, const void* v,
                         const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* dq,
                         void* dk, void* dv, float* d_ts_weights, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return logged("hstu_jagged_attn_bwd", p, hstu_jagged_attn_bwd_body(p, dout, q, k, v, offsets, timestamps, ts_weights, dq, dk, dv, d_ts_weights, workspace, workspace_bytes, stream));
}

int hstu_jagged_attn_fwd_noalloc(const hstu_problem_t* p, const void* q, const void* k, const void* v,
                                 const int64_t* offsets, const int64_t* timestamps, const void* ts_weights, void* out,
                                 void* stream) {
  return logged("hstu_jagged_attn_fwd_noalloc", p, hstu_jagged_attn_fwd_noalloc_body(p, q, k, v, offsets, timestamps, ts_weights, out, stream));
}

int hstu_sl_select(const int64_t* offsets, int64_t num_seqs, int64_t total_rows, int64_t max_seq_len, double alpha,
                   const float* seq_uniform, const uint32_t* token_keys, int64_t* out_offsets, int64_t* out_index,
                   void* stream) {
  return logged("hstu_sl_select", nullptr, hstu_sl_select_body(offsets, num_seqs, total_rows, max_seq_len, alpha, seq_uniform, token_keys, out_offsets, out_index, stream));
}

int hstu_gather_rows(const void* in, void* out, int64_t row_bytes, const int64_t* index, const int64_t* count,
                     int64_t max_rows, void* stream) {
  return logged("hstu_gather_rows", nullptr, hstu_gather_rows_body(in, out, row_bytes, index, count, max_rows, stream));
}

int hstu_layer_projection(const void* x, const void* w, int64_t total_rows, int64_t d_model, int64_t num_heads,
                          int64_t d_qk, int64_t d_v, void* u, void* v, void* q, void* k, void* stream) {
  return logged("hstu_layer_projection", nullptr, hstu_layer_projection_body(x, w, total_rows, d_model, num_heads, d_qk, d_v, u, v, q, k, stream));
}

int hstu_layer_norm_gate(const void* o, const void* u, void* y, int64_t total_rows, int64_t width, double eps,
                         void* stream) {
  return logged("hstu_layer_norm_gate", nullptr, hstu_layer_norm_gate_body(o, u, y, total_rows, width, eps, stream));
}

int hstu_cp_reorder(const void* in, void* out, int64_t row_bytes, const int64_t* offsets, int64_t num_seqs,
                    int64_t total_rows, int64_t max_seq_len, int64_t cp_size, int inverse, int64_t* out_offsets,
                    void* stream) {
  return logged("hstu_cp_reorder", nullptr, hstu_cp_reorder_body(in, out, row_bytes, offsets, num_seqs, total_rows, max_seq_len, cp_size, inverse, out_offsets, stream));
}
