// HSTU layer steps either side of the attention (Actions Speak Louder than
// Words, §3: a layer is a pointwise projection, the spatial aggregation, and a
// pointwise transformation; the interaction is Norm(A(X)V(X)) ⊙ U(X)).
//
//   proj_kernel       [U V Q K] = SiLU(X Wᵀ): X [T, Dm], W [N, Dm] (a linear
//                     layer's weight layout), N = H (2 d_v + 2 d_qk); one MFMA
//                     GEMM with the SiLU and the split into the four outputs
//                     fused into its store.
//   norm_gate_kernel  Y = LayerNorm(O) ⊙ U per row of H d_v values (fp32
//                     statistics, no learned scale or shift).
#include <hip/hip_runtime.h>

#include "layer.h"
#include "swtile.h"

namespace hstu {

namespace {

constexpr int kProjThreads = 256;  // 4 waves
constexpr int kTM = 128;           // rows of X per tile
constexpr int kTN = 128;           // columns of the projection per tile
constexpr int kTK = 64;            // contraction step (elements of Dm)

struct alignas(16) ProjSmem {
  __bf16 x[2][kTM * kTK];  // X rows of the step, swizzled (SwTile<bf16, 64>)
  __bf16 w[2][kTN * kTK];  // W rows (output columns) of the step
};

// Tile (tn, tm): output columns [128 tn, +128) for rows [128 tm, +128).  Wave
// w computes columns 64 (w >> 1) .. +63 for rows 64 (w & 1) .. +63 as a 2 x 2
// set of 32 x 32 MFMA blocks, transposed (D[n][t] = sum_k W[n][k] X[t][k]) so
// that each lane holds one row t: lane (r32, g) of block (j, i) holds row
// 64 (w & 1) + 32 i + r32, columns 64 (w >> 1) + 32 j + acc_row(e, g).
__global__ __launch_bounds__(kProjThreads, 2) void proj_kernel(const ProjParams p) {
  __shared__ ProjSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tn = blockIdx.x, tm = blockIdx.y;
  const int64_t row0 = (int64_t)tm * kTM;
  const int nvalid = (int)min<int64_t>(kTM, p.T - row0);
  const int col0 = tn * kTN;
  const __bf16* X = static_cast<const __bf16*>(p.x) + row0 * p.Dm;
  const __bf16* W = static_cast<const __bf16*>(p.w) + (int64_t)col0 * p.Dm;
  const uint32_t lane_off = tile_lane_offset<__bf16, kTK, kProjThreads>(tid, p.Dm);
  LaneOffsets<kTK> lo;
  lo.init(lane);
  const int tb = wave & 1, nb = wave >> 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[j][i] = f32x16{};
  const int nk = (int)(p.Dm / kTK);
  tile_load_async<__bf16, kTK, kTM, kProjThreads>(sm.x[0], X, p.Dm, nvalid, tid, lane_off);
  tile_load_async<__bf16, kTK, kTN, kProjThreads>(sm.w[0], W, p.Dm, kTN, tid, lane_off);
  wait_loads();
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) {
      tile_load_async<__bf16, kTK, kTM, kProjThreads>(sm.x[cur ^ 1], X + (ks + 1) * kTK, p.Dm, nvalid, tid, lane_off);
      tile_load_async<__bf16, kTK, kTN, kProjThreads>(sm.w[cur ^ 1], W + (ks + 1) * kTK, p.Dm, kTN, tid, lane_off);
    }
    const char* xb = reinterpret_cast<const char*>(sm.x[cur]);
    const char* wb = reinterpret_cast<const char*>(sm.w[cur]);
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        a[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wb + lo.row[kk] + (nb * 2 + j) * 32 * kTK * 2));
#pragma unroll
      for (int i = 0; i < 2; ++i)
        b[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xb + lo.row[kk] + (tb * 2 + i) * 32 * kTK * 2));
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[j][i] = Mma<__bf16>::mma(a[j], b[i], acc[j][i]);
    }
    wait_loads();
    __syncthreads();
  }
  // SiLU and the store into the section this tile's columns belong to (each
  // section's width is a multiple of the tile width, so one per tile)
  int sec = 0, c = col0;
  while (sec < 3 && c >= p.width[sec]) c -= p.width[sec++];
  __bf16* out = static_cast<__bf16*>(p.out[sec]);
  const int64_t ld = p.width[sec];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = tb * 64 + i * 32 + r32;
    if (t >= nvalid) continue;
    __bf16* dst = out + (row0 + t) * ld + c + nb * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[j][i][4 * qd + e];
          v[e] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
        }
        const int n = j * 32 + 8 * qd + 4 * g;
        *reinterpret_cast<u32x2*>(dst + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}

constexpr int kNormThreads = 256;  // one wave per row

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// One wave per row of `width` bf16 values (width a multiple of 8, at most
// 64 x 8 x kNormChunks): each lane holds whole 16-byte chunks.
constexpr int kNormChunks = 8;

template <int CH>  // 16-byte chunks per lane: the row width is at most 64 x 8 x CH
__global__ __launch_bounds__(kNormThreads) void norm_gate_kernel(const __bf16* __restrict__ o,
                                                                 const __bf16* __restrict__ u,
                                                                 __bf16* __restrict__ y, int64_t T, int width,
                                                                 float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nchunks = width / 8;
  const u32x4* orow = reinterpret_cast<const u32x4*>(o + t * width);
  const u32x4* urow = reinterpret_cast<const u32x4*>(u + t * width);
  u32x4* yrow = reinterpret_cast<u32x4*>(y + t * width);
  // both rows are loaded up front, so that the U row's latency passes during
  // the two reductions
  float x[CH][8];
  bf16x8 gate[CH];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int ch = lane + 64 * j;
    if (ch < nchunks) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(orow + ch));
      gate[j] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(urow + ch));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[j][e] = (float)v[e];
        sum += x[j][e];
      }
    }
  }
  const float mean = wave_sum(sum) / (float)width;
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    if (lane + 64 * j < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dlt = x[j][e] - mean;
        sq += dlt * dlt;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)width + eps);
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int ch = lane + 64 * j;
    if (ch < nchunks) {
      const bf16x8 g = gate[j];
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (x[j][e] - mean) * rstd * (float)g[e];
      __builtin_nontemporal_store(u32x4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                                        pack_bf16x2(r[6], r[7])},
                                  yrow + ch);
    }
  }
}

}  // namespace

int proj_tile_rows() { return kTM; }
int proj_tile_cols() { return kTN; }
int proj_tile_k() { return kTK; }
int norm_max_width() { return 64 * 8 * kNormChunks; }

hipError_t launch_proj(const ProjParams& p, hipStream_t s) {
  const unsigned nt = (unsigned)((p.T + kTM - 1) / kTM);
  hipLaunchKernelGGL(proj_kernel, dim3((unsigned)(p.N / kTN), nt), dim3(kProjThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_norm_gate(const void* o, const void* u, void* y, int64_t T, int width, float eps, hipStream_t s) {
  const int64_t blocks = (T + (kNormThreads / 64) - 1) / (kNormThreads / 64);
  // the fewest chunks per lane that hold the row: registers (and so the
  // waves in flight) follow the row width
  const int per_lane = (width / 8 + 63) / 64;
  const auto k = per_lane <= 1 ? norm_gate_kernel<1>
                 : per_lane <= 2 ? norm_gate_kernel<2>
                 : per_lane <= 4 ? norm_gate_kernel<4>
                                 : norm_gate_kernel<kNormChunks>;
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kNormThreads), 0, s, static_cast<const __bf16*>(o),
                     static_cast<const __bf16*>(u), static_cast<__bf16*>(y), T, width, eps);
  return hipGetLastError();
}

}  // namespace hstu
