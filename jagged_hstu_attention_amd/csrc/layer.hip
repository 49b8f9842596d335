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

// XCD-aware tile order.  The dispatcher hands consecutive workgroups to the
// chip's kXcds L2 domains in turn, so workgroup b runs on domain b % kXcds.
// The column tiles of one row block are given to consecutive workgroups of
// one domain: they run there at about the same time and read that block's X
// rows from one L2 copy (W, a few MB, stays resident in every domain's L2).
// Row block tm belongs to domain tm % kXcds.
constexpr int kXcds = 8;

__host__ __device__ inline int64_t proj_row_blocks(int64_t T) { return (T + kTM - 1) / kTM; }
__host__ __device__ inline int64_t proj_grid(int64_t T, int64_t N) {
  return (proj_row_blocks(T) + kXcds - 1) / kXcds * kXcds * (N / kTN);
}

// Tile (tn, tm): output columns [128 tn, +128) for rows [128 tm, +128).  Wave
// w computes columns 64 (w >> 1) .. +63 for rows 64 (w & 1) .. +63 as a 2 x 2
// set of 32 x 32 MFMA blocks, transposed (D[n][t] = sum_k W[n][k] X[t][k]) so
// that each lane holds one row t: lane (r32, g) of block (j, i) holds row
// 64 (w & 1) + 32 i + r32, columns 64 (w >> 1) + 32 j + acc_row(e, g).
__global__ __launch_bounds__(kProjThreads, 2) void proj_kernel(const ProjParams p) {
  // The two buffers of each operand are separate LDS arrays and every step
  // names its buffers at compile time (the step loop runs two steps per
  // turn): the compiler then knows that a step's reads of its current tiles
  // do not touch the next tiles' direct-to-LDS writes, and inserts no wait for
  // those loads before the reads.  One shared array indexed by the step
  // parity would make every step wait for its own prefetch.
  __shared__ __attribute__((aligned(16))) __bf16 xs0[kTM * kTK], xs1[kTM * kTK];
  __shared__ __attribute__((aligned(16))) __bf16 ws0[kTN * kTK], ws1[kTN * kTK];
  const int tid = threadIdx.x, lane = tid & 63, r32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nct = (int)(p.N / kTN);
  const int xcd = (int)(blockIdx.x % kXcds), turn = (int)(blockIdx.x / kXcds);
  const int tn = turn % nct;
  const int64_t tm = (int64_t)(turn / nct) * kXcds + xcd;
  if (tm >= proj_row_blocks(p.T)) return;  // the last turns of a domain past the row blocks
  const int64_t row0 = tm * kTM;
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
  tile_load_async<__bf16, kTK, kTM, kProjThreads>(xs0, X, p.Dm, nvalid, tid, lane_off);
  tile_load_async<__bf16, kTK, kTN, kProjThreads>(ws0, W, p.Dm, kTN, tid, lane_off);
  wait_loads();
  __syncthreads();
  static_assert(tile_load_steps<__bf16, kTK, kTM, kProjThreads>() == kTK / 16 &&
                    tile_load_steps<__bf16, kTK, kTN, kProjThreads>() == kTK / 16,
                "one load of each next tile per contraction slice");
  // One contraction step over the tiles (xc, wc); the next step's tiles are
  // loaded into (xn, wn) one instruction per slice, after the slice's MFMAs,
  // so that each load's issue overlaps MFMAs already in the pipe.
  const auto step = [&](const __bf16* xc, const __bf16* wc, __bf16* xn, __bf16* wn, int ks) {
    const bool more = ks + 1 < nk;
    const char* xb = reinterpret_cast<const char*>(xc);
    const char* wb = reinterpret_cast<const char*>(wc);
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
      if (more) {
        tile_load_step<__bf16, kTK, kTM, kProjThreads>(xn, X + (ks + 1) * kTK, p.Dm, nvalid, tid, lane_off, kk);
        tile_load_step<__bf16, kTK, kTN, kProjThreads>(wn, W + (ks + 1) * kTK, p.Dm, kTN, tid, lane_off, kk);
      }
    }
    wait_loads();
    __syncthreads();
  };
  for (int ks = 0; ks < nk; ks += 2) {
    step(xs0, ws0, xs1, ws1, ks);
    if (ks + 1 < nk) step(xs1, ws1, xs0, ws0, ks + 1);
  }
  // SiLU and the store into the section this tile's columns belong to (each
  // section's width is a multiple of the tile width, so one per tile).  A
  // lane holds one output row, so stores straight from the accumulators
  // would write 8 bytes to each of 64 rows per instruction.  Each wave
  // instead stages its 64 x 64 block in LDS (the step buffers are free after
  // the last step's barrier; 8 KB per wave, 16-byte chunks XOR-swizzled by
  // row so that the writes and the row reads spread over the banks) and
  // stores whole 128-byte row segments, 8 rows per instruction.
  int sec = 0, c = col0;
  while (sec < 3 && c >= p.width[sec]) c -= p.width[sec++];
  __bf16* out = static_cast<__bf16*>(p.out[sec]);
  const int64_t ld = p.width[sec];
  char* stg = reinterpret_cast<char*>(wave < 2 ? xs0 : xs1) + (wave & 1) * 8192;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = i * 32 + r32;  // row within the wave's block
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
        // columns j*32 + 8 qd + 4 g .. +3: half g of 16-byte chunk 4 j + qd
        const int ch = (4 * j + qd) ^ (t & 7);
        *reinterpret_cast<u32x2*>(stg + t * 128 + ch * 16 + g * 8) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
  const int cq = lane & 7;  // the 16-byte chunk this lane stores
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int t = 8 * k + (lane >> 3);
    const u32x4 val = *reinterpret_cast<const u32x4*>(stg + t * 128 + (cq ^ (t & 7)) * 16);
    const int tt = tb * 64 + t;
    if (tt < nvalid)
      *reinterpret_cast<u32x4*>(out + (row0 + tt) * ld + c + nb * 64 + cq * 8) = val;
  }
}

constexpr int kNormThreads = 256;  // one wave per row

// Sum over the wave: row sums by DPP moves (two quad permutations, then the
// half-row and row mirrors; every lane of a row ends with the same sum), then
// the four rows' sums read into scalars.  No LDS round trip.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int o;
  const int x = __builtin_bit_cast(int, v);
  switch (ctrl_sel) {
    case 0: o = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // lane ^ 1
    case 1: o = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // lane ^ 2
    case 2: o = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // 7 - i within 8 lanes
    default: o = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break; // 15 - i within the row
  }
  return v + __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v = dpp_add(v, k);
  const int x = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48));
  return (r0 + r1) + (r2 + r3);
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
int64_t proj_workgroups(int64_t T, int64_t N) { return proj_grid(T, N); }

hipError_t launch_proj(const ProjParams& p, hipStream_t s) {
  hipLaunchKernelGGL(proj_kernel, dim3((unsigned)proj_grid(p.T, p.N)), dim3(kProjThreads), 0, s, p);
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
