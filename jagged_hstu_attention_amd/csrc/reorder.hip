// Load-balanced chunk-pair reorder (Scaling Generative Recommendations with
// Context Parallelism on HSTU, §2.3: each sequence is cut into 2C mini-chunks,
// rank r takes chunks r and 2C-1-r, and a memory-reordering kernel lays the
// data out per rank instead of chunking and concatenating).
//
// Rank-major layout: for r in [0, C), for b in [0, B): the rows of mini-chunk r
// of sequence b, then those of mini-chunk 2C-1-r.  Chunk k of a length-L
// sequence is rows [floor(kL/2C), floor((k+1)L/2C)).  For one (r, b) the two
// chunks are contiguous runs in the sequence-major layout and one contiguous run
// in the rank-major layout, so the kernel is a set of contiguous byte copies:
// workgroup (pair, slice) copies one slice of one (r, b) pair with the widest
// vector width the row size and pointers allow.  Bytes are never interpreted,
// so the result is bit-exact whatever the element type.
#include "attn.h"

namespace hstu {

namespace {

constexpr int kReorderThreads = 256;
constexpr int64_t kSliceBytes = 64 * 1024;

// floor(k L / nch) for 0 <= k <= nch <= 2048 and L < 2^42: k L is an exact
// double, the quotient is correctly rounded (error below 2^-11 for a quotient
// under 2^42), and a non-integral quotient lies at least 1/nch >= 2^-11 below
// the next integer, so the floor is exact.  A 64-bit integer division would
// take a long software loop.
__device__ __forceinline__ int64_t chunk_lo64(int64_t L, int64_t k, int64_t nch) {
  return (int64_t)floor((double)(k * L) / (double)nch);
}

// Rows of sequence b (length L) held by ranks < r: floor(rL/2C) + L - floor((2C-r)L/2C).
__device__ __forceinline__ int64_t rows_before_rank(int64_t L, int64_t r, int64_t nch) {
  return chunk_lo64(L, r, nch) + L - chunk_lo64(L, nch - r, nch);
}

__device__ __forceinline__ int64_t pair_rows(int64_t L, int64_t r, int64_t nch) {
  const int64_t c1 = nch - 1 - r;
  return (chunk_lo64(L, r + 1, nch) - chunk_lo64(L, r, nch)) + (chunk_lo64(L, c1 + 1, nch) - chunk_lo64(L, c1, nch));
}

template <typename V>
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(const char* __restrict__ in, char* __restrict__ out,
                                                                  int64_t rb, const int64_t* __restrict__ offsets,
                                                                  int64_t B, int64_t T, int64_t C, int inverse,
                                                                  int64_t* __restrict__ out_offsets) {
  __shared__ int64_t wave_part[kReorderThreads / 64];
  const int64_t pair = blockIdx.x;
  const int64_t r = pair / B, b = pair % B;
  const int64_t nch = 2 * C;
  const int tid = threadIdx.x;

  // Start of segment (r, b) in the rank-major layout: all rows of ranks < r,
  // plus rank r's rows of sequences < b.  The workgroup sums the sequences
  // with a stride (each thread B / 256 of them), then reduces across waves.
  int64_t part = 0;
  for (int64_t bb = tid; bb < B; bb += kReorderThreads) {
    const int64_t Lb = offsets[bb + 1] - offsets[bb];
    part += rows_before_rank(Lb, r, nch);
    if (bb < b) part += pair_rows(Lb, r, nch);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) wave_part[tid >> 6] = part;
  __syncthreads();
  int64_t start = 0;
#pragma unroll
  for (int w = 0; w < kReorderThreads / 64; ++w) start += wave_part[w];

  const int64_t o0 = offsets[b];
  const int64_t L = offsets[b + 1] - o0;
  const int64_t c1 = nch - 1 - r;
  const int64_t a0 = chunk_lo64(L, r, nch), alen = chunk_lo64(L, r + 1, nch) - a0;
  const int64_t b0 = chunk_lo64(L, c1, nch), blen = chunk_lo64(L, c1 + 1, nch) - b0;
  if (blockIdx.y == 0 && tid == 0 && out_offsets) {
    out_offsets[pair] = start;
    if (pair == C * B - 1) out_offsets[C * B] = T;
  }

  const int64_t bytes = (alen + blen) * rb;
  const int64_t lo = (int64_t)blockIdx.y * kSliceBytes;
  if (lo >= bytes) return;
  const int64_t hi = lo + kSliceBytes < bytes ? lo + kSliceBytes : bytes;
  const int64_t abytes = alen * rb;
  const char* rank_base_in = in + start * rb;           // rank-major side (inverse)
  char* rank_base_out = out + start * rb;               // rank-major side (forward)
  const int64_t seg_a = (o0 + a0) * rb, seg_b = (o0 + b0) * rb;

  // Each thread moves kU vectors per round; the data is streamed once, so the
  // accesses are non-temporal.
  constexpr int kU = 8;
  constexpr int64_t kStep = (int64_t)kReorderThreads * sizeof(V);
  for (int64_t x0 = lo + tid * (int64_t)sizeof(V); x0 < hi; x0 += kU * kStep) {
    V val[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t x = x0 + u * kStep;
      if (x < hi) {
        const int64_t seq_off = x < abytes ? seg_a + x : seg_b + (x - abytes);
        const V* src = inverse ? reinterpret_cast<const V*>(rank_base_in + x) : reinterpret_cast<const V*>(in + seq_off);
        val[u] = __builtin_nontemporal_load(src);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t x = x0 + u * kStep;
      if (x < hi) {
        const int64_t seq_off = x < abytes ? seg_a + x : seg_b + (x - abytes);
        V* dst = inverse ? reinterpret_cast<V*>(out + seq_off) : reinterpret_cast<V*>(rank_base_out + x);
        __builtin_nontemporal_store(val[u], dst);
      }
    }
  }
}

}  // namespace

hipError_t launch_reorder(const void* in, void* out, int64_t row_bytes, const int64_t* offsets, int64_t B,
                          int64_t total_rows, int64_t max_seq_len, int cp_size, bool inverse,
                          int64_t* out_offsets, hipStream_t s) {
  const int64_t nch = 2 * (int64_t)cp_size;
  // Largest pair: two chunks of at most ceil(L/2C) rows each.
  const int64_t max_pair_rows = 2 * ((max_seq_len + nch - 1) / nch);
  const int64_t max_pair_bytes = max_pair_rows * row_bytes;
  int64_t slices = (max_pair_bytes + kSliceBytes - 1) / kSliceBytes;
  if (slices < 1) slices = 1;
  const dim3 grid((unsigned)(cp_size * B), (unsigned)slices);
  const uintptr_t align = (uintptr_t)in | (uintptr_t)out | (uintptr_t)row_bytes;
  const char* i = static_cast<const char*>(in);
  char* o = static_cast<char*>(out);
  const int inv = inverse ? 1 : 0;
  if ((align & 15) == 0)
    hipLaunchKernelGGL(reorder_kernel<u32x4>, grid, dim3(kReorderThreads), 0, s, i, o, row_bytes, offsets, B,
                       total_rows, (int64_t)cp_size, inv, out_offsets);
  else if ((align & 7) == 0)
    hipLaunchKernelGGL(reorder_kernel<u32x2>, grid, dim3(kReorderThreads), 0, s, i, o, row_bytes, offsets, B,
                       total_rows, (int64_t)cp_size, inv, out_offsets);
  else if ((align & 3) == 0)
    hipLaunchKernelGGL(reorder_kernel<uint32_t>, grid, dim3(kReorderThreads), 0, s, i, o, row_bytes, offsets, B,
                       total_rows, (int64_t)cp_size, inv, out_offsets);
  else
    hipLaunchKernelGGL(reorder_kernel<uint8_t>, grid, dim3(kReorderThreads), 0, s, i, o, row_bytes, offsets, B,
                       total_rows, (int64_t)cp_size, inv, out_offsets);
  return hipGetLastError();
}

}  // namespace hstu
