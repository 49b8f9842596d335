// Stochastic Length (Actions Speak Louder than Words, §3.2 and §4.2: long
// histories are sparsified by keeping a subsequence; at alpha = 1.6 a
// length-4096 history becomes length 776 most of the time; App. E: the
// subsequence is chosen by recency or at random, among others).
//
// A sequence of length n is cut to L = floor(n^(alpha/2)) rows unless its
// draw u (an input in [0, 1)) falls below n^(alpha-2), in which case it is
// kept whole.  The kept rows are the last L (recency) or the L rows with the
// smallest random keys (an input per row), equal keys taken in position
// order; either way they stay in their original order.  Three kernels:
//   sl_lengths_kernel  one workgroup: every sequence's kept length and the
//                      exclusive scan of them (the output offsets);
//   sl_select_kernel   one workgroup per sequence: the input row of every
//                      output row (radix select of the L-th key, then an
//                      order-preserving compaction);
//   gather_rows_kernel out[i] = in[index[i]] for the rows the offsets count,
//                      any row size, bytes copied unchanged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sl.h"

namespace hstu {

namespace {

constexpr int kLenThreads = 1024;
constexpr int kSelThreads = 256;

// floor(n^(alpha/2)) from the double-precision power; the factor 1 + 2^-40
// keeps a power that is an exact integer from landing one ulp below it.
__device__ __forceinline__ int64_t sl_length(int64_t n, double alpha) {
  if (n <= 0) return 0;
  const double x = pow((double)n, 0.5 * alpha) * (1.0 + 0x1p-40);
  const int64_t L = (int64_t)floor(x);
  return L < n ? L : n;
}

__device__ __forceinline__ int64_t kept_length(int64_t n, double alpha, float u) {
  const int64_t L = sl_length(n, alpha);
  if (n <= 1 || L >= n) return n;
  return (double)u < pow((double)n, alpha - 2.0) ? n : L;
}

__global__ __launch_bounds__(kLenThreads) void sl_lengths_kernel(const int64_t* __restrict__ offsets, int64_t B,
                                                                 double alpha, const float* __restrict__ u,
                                                                 int64_t* __restrict__ out_offsets) {
  __shared__ int64_t wsum[kLenThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < B; base += kLenThreads) {
    const int64_t b = base + t;
    const int64_t m = b < B ? kept_length(offsets[b + 1] - offsets[b], alpha, u[b]) : 0;
    int64_t incl = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int64_t before = 0, all = 0;
    for (int i = 0; i < kLenThreads / 64; ++i) {
      before += i < wave ? wsum[i] : 0;
      all += wsum[i];
    }
    if (b < B) out_offsets[b] = carry + before + incl - m;
    carry += all;
    __syncthreads();
  }
  if (t == 0) out_offsets[B] = carry;
}

// Exclusive scan of one 32-bit value per thread over the workgroup (kSelThreads
// threads); total in *total.
__device__ __forceinline__ uint32_t scan_sel(uint32_t v, uint32_t* buf, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    before += i < wave ? buf[i] : 0;
    all += buf[i];
  }
  *total = all;
  __syncthreads();
  return before + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void sl_select_kernel(const int64_t* __restrict__ offsets,
                                                                const int64_t* __restrict__ out_offsets,
                                                                const uint32_t* __restrict__ keys,
                                                                int64_t* __restrict__ index) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sbuf[kSelThreads / 64];
  __shared__ uint32_t s_prefix, s_need;
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t lo = offsets[b], n = offsets[b + 1] - lo;
  const int64_t o = out_offsets[b], m = out_offsets[b + 1] - o;
  if (m <= 0) return;
  if (m == n || !keys) {
    // kept whole, or recency: the last m rows
    for (int64_t j = t; j < m; j += kSelThreads) index[o + j] = lo + (n - m) + j;
    return;
  }
  const uint32_t* k = keys + lo;
  // Radix select, 8 bits per pass from the top: after the passes, `prefix`
  // is the m-th smallest key and `need` how many rows with that key are kept.
  uint32_t prefix = 0, need = (uint32_t)m;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
    const uint32_t himask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int64_t j = t; j < n; j += kSelThreads) {
      const uint32_t x = k[j];
      if ((x & himask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    // the digit holding the need-th smallest key: one bin per thread, an
    // exclusive scan of the counts, and the one bin whose range [before,
    // before + count) contains need - 1 publishes it
    static_assert(kSelThreads == 256, "one histogram bin per thread");
    const uint32_t c = hist[t];
    uint32_t all;
    const uint32_t before = scan_sel(c, sbuf, &all);
    if (before < need && need <= before + c) {
      s_prefix = prefix | ((uint32_t)t << shift);
      s_need = need - before;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    __syncthreads();
  }
  // Order-preserving compaction: a row is kept if its key is below the
  // threshold key, or equal to it and among the first `need` such rows.  The
  // rows kept before row j are the smaller keys before it and the first
  // min(#equal keys before it, need) equal ones, so one scan of both counts
  // (smaller in the low half, equal in the high half: at most kSelThreads
  // each per chunk) places every kept row.
  uint32_t lt_before = 0, eq_before = 0;
  for (int64_t base = 0; base < n; base += kSelThreads) {
    const int64_t j = base + t;
    const uint32_t x = j < n ? k[j] : 0xFFFFFFFFu;
    const uint32_t lt = j < n && x < prefix ? 1u : 0u;
    const uint32_t eq = j < n && x == prefix ? 1u : 0u;
    uint32_t total;
    const uint32_t pre = scan_sel(lt | (eq << 16), sbuf, &total);
    const uint32_t lt_rank = lt_before + (pre & 0xFFFFu), eq_rank = eq_before + (pre >> 16);
    if (lt || (eq && eq_rank < need)) index[o + lt_rank + min(eq_rank, need)] = lo + j;
    lt_before += total & 0xFFFFu;
    eq_before += total >> 16;
  }
}

// Rows copied as vectors of V bytes; the row count is read on the device.
template <typename V>
__global__ void gather_rows_kernel(const char* __restrict__ in, char* __restrict__ out, int64_t row_vecs,
                                   const int64_t* __restrict__ index, const int64_t* __restrict__ count,
                                   int64_t max_rows) {
  const int64_t rows = min(*count, max_rows);
  const int64_t total = rows * row_vecs;
  const V* src = reinterpret_cast<const V*>(in);
  V* dst = reinterpret_cast<V*>(out);
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / row_vecs, c = v - r * row_vecs;
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + index[r] * row_vecs + c), dst + v);
  }
}

}  // namespace

hipError_t launch_sl_select(const int64_t* offsets, int64_t B, double alpha, const float* seq_uniform,
                            const uint32_t* token_keys, int64_t* out_offsets, int64_t* out_index, hipStream_t s) {
  hipLaunchKernelGGL(sl_lengths_kernel, dim3(1), dim3(kLenThreads), 0, s, offsets, B, alpha, seq_uniform,
                     out_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sl_select_kernel, dim3((unsigned)B), dim3(kSelThreads), 0, s, offsets, out_offsets, token_keys,
                     out_index);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* in, void* out, int64_t row_bytes, const int64_t* index,
                              const int64_t* count, int64_t max_rows, int vec_bytes, int cus, hipStream_t s) {
  const int64_t row_vecs = row_bytes / vec_bytes;
  const int64_t total = max_rows * row_vecs;
  constexpr int kThreads = 256;
  const int64_t want = (total + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < (int64_t)cus * 16 ? (want > 0 ? want : 1) : (int64_t)cus * 16);
  const char* i = static_cast<const char*>(in);
  char* o = static_cast<char*>(out);
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  switch (vec_bytes) {
    case 16: hipLaunchKernelGGL(gather_rows_kernel<v4u>, dim3(grid), dim3(kThreads), 0, s, i, o, row_vecs, index,
                                count, max_rows); break;
    case 8: hipLaunchKernelGGL(gather_rows_kernel<v2u>, dim3(grid), dim3(kThreads), 0, s, i, o, row_vecs, index,
                               count, max_rows); break;
    case 4: hipLaunchKernelGGL(gather_rows_kernel<uint32_t>, dim3(grid), dim3(kThreads), 0, s, i, o, row_vecs, index,
                               count, max_rows); break;
    default: hipLaunchKernelGGL(gather_rows_kernel<uint8_t>, dim3(grid), dim3(kThreads), 0, s, i, o, row_vecs, index,
                                count, max_rows); break;
  }
  return hipGetLastError();
}

}  // namespace hstu
