// LDS staging and MFMA tile helpers for the attention kernels.
#pragma once

#include "common.h"

namespace hstu {

// Padded LDS pitches (in elements).  Row-major tiles get 16 extra bytes per row
// so that the 32 lanes reading one column slice of 32 consecutive rows hit
// distinct banks; transposed bf16 tiles likewise.
template <typename T, int D> struct Pitch {
  static constexpr int row = D + 16 / (int)sizeof(T);
};
template <int ROWS> struct TPitch {
  static constexpr int col = ROWS + 8;  // bf16 elements
};

// Copy `ROWS` rows of D elements (row r at src + r*ld) into a row-major LDS
// tile; rows >= nvalid are zero-filled.  16-byte accesses.
template <typename T, int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows(T* __restrict__ dst, const T* __restrict__ src, int64_t ld,
                                           int nvalid, int tid) {
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kPerRow = D / kVec;
  constexpr int kTotal = ROWS * kPerRow;
  constexpr int kPitch = Pitch<T, D>::row;
#pragma unroll
  for (int c = tid; c < kTotal; c += NT) {
    const int r = c / kPerRow, col = (c % kPerRow) * kVec;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nvalid) val = *reinterpret_cast<const u32x4*>(src + r * ld + col);
    *reinterpret_cast<u32x4*>(dst + r * kPitch + col) = val;
  }
}

// Copy ROWS rows of D bf16 into a transposed LDS tile dst[col][slot(row)]
// (see tslot).  Each task moves a 4-row x 8-column block: four 16-byte global
// loads, byte permutes, eight 8-byte LDS stores.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void stage_rows_t(__bf16* __restrict__ dst, const __bf16* __restrict__ src,
                                             int64_t ld, int nvalid, int tid) {
  constexpr int kTasks = (ROWS / 4) * (D / 8);
  constexpr int kTP = TPitch<ROWS>::col;
#pragma unroll
  for (int t = tid; t < kTasks; t += NT) {
    const int rq = t % (ROWS / 4), dc = t / (ROWS / 4);
    u32x4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = rq * 4 + j;
      r[j] = u32x4{0u, 0u, 0u, 0u};
      if (row < nvalid) r[j] = *reinterpret_cast<const u32x4*>(src + row * ld + dc * 8);
    }
    __bf16* base = dst + (dc * 8) * kTP + tslot(rq * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(r[1][e >> 1], r[0][e >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(r[3][e >> 1], r[2][e >> 1], sel);
      *reinterpret_cast<u32x2*>(base + e * kTP) = u32x2{lo, hi};
    }
  }
}

// acc (32 tile-rows x 32 lanes) = sum over d of tile[row][d] * op[d] where
// `tile` is row-major (A operand) and `op` holds this lane's B-operand slices.
template <typename T, int D>
__device__ __forceinline__ f32x16 mma_tile_rows(const T* __restrict__ tile, int row,
                                                const typename Mma<T>::operand* op, int g) {
  using M = Mma<T>;
  constexpr int kPitch = Pitch<T, D>::row;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / M::kK; ++kk)
    acc = M::mma(M::load(tile + row * kPitch + kk * M::kK + g * M::kEpl), op[kk], acc);
  return acc;
}

// out[dblk] += sum over the ROWS contraction rows of X[row][d] * vals[row] where
// vals come as accumulator fragments (vals[blk][i] belongs to contraction row
// blk*32 + acc_row(i, g)).  bf16: X is a transposed tile; fp32: X is row-major.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void mma_contract_rows(f32x16* out, const T* __restrict__ X,
                                                  const float (*vals)[16], int r32, int g) {
  using M = Mma<T>;
  if constexpr (sizeof(T) == 2) {
    constexpr int kTP = TPitch<ROWS>::col;
    bf16x8 b[ROWS / 32][2];
#pragma unroll
    for (int blk = 0; blk < ROWS / 32; ++blk)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) b[blk][u][j] = (__bf16)vals[blk][8 * u + j];
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int blk = 0; blk < ROWS / 32; ++blk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          out[dblk] = M::mma(M::load(X + (dblk * 32 + r32) * kTP + blk * 32 + 16 * u + 8 * g), b[blk][u],
                             out[dblk]);
  } else {
    constexpr int kPitch = Pitch<T, D>::row;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int blk = 0; blk < ROWS / 32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          out[dblk] = M::mma(X[(blk * 32 + acc_row(i, g)) * kPitch + dblk * 32 + r32], vals[blk][i], out[dblk]);
  }
}

// Store an accumulator block set out[dblk] (rows = d, column = this lane's row)
// to dst[0..D) of one row, converting to T.
template <typename T, int D>
__device__ __forceinline__ void store_row_from_acc(T* __restrict__ dst, const f32x16* acc, int g) {
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = dblk * 32 + qd * 8 + 4 * g;
      if constexpr (sizeof(T) == 2) {
        u32x2 v = {pack_bf16x2(acc[dblk][4 * qd], acc[dblk][4 * qd + 1]),
                   pack_bf16x2(acc[dblk][4 * qd + 2], acc[dblk][4 * qd + 3])};
        *reinterpret_cast<u32x2*>(dst + d0) = v;
      } else {
        float4 v = {acc[dblk][4 * qd], acc[dblk][4 * qd + 1], acc[dblk][4 * qd + 2], acc[dblk][4 * qd + 3]};
        *reinterpret_cast<float4*>(dst + d0) = v;
      }
    }
}

}  // namespace hstu

namespace hstu {

// Register-staged copy of ROWS x D elements (row r at src + r*ld) into a
// row-major LDS tile, split in a global-load half (issued one tile ahead) and
// an LDS-store half.  Rows >= nvalid are zero-filled.
template <typename T, int D, int ROWS, int NT> struct RowStage {
  static constexpr int kVec = 16 / sizeof(T);
  static constexpr int kPerRow = D / kVec;
  static constexpr int kTotal = ROWS * kPerRow;
  static constexpr int kIters = (kTotal + NT - 1) / NT;
  u32x4 r[kIters];
  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t ld, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int c = tid + it * NT;
      const int row = c / kPerRow, col = (c % kPerRow) * kVec;
      r[it] = u32x4{0u, 0u, 0u, 0u};
      if (c < kTotal && row < nvalid) r[it] = *reinterpret_cast<const u32x4*>(src + row * ld + col);
    }
  }
  __device__ __forceinline__ void store(T* __restrict__ dst, int tid) const {
    constexpr int kPitch = Pitch<T, D>::row;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int c = tid + it * NT;
      const int row = c / kPerRow, col = (c % kPerRow) * kVec;
      if (c < kTotal) *reinterpret_cast<u32x4*>(dst + row * kPitch + col) = r[it];
    }
  }
};

// Register-staged transposed copy (bf16): each task is a 4-row x 8-column
// block, stored as eight 8-byte runs of the transposed tile (see tslot).
template <int D, int ROWS, int NT> struct TStage {
  static constexpr int kTasks = (ROWS / 4) * (D / 8);
  static constexpr int kIters = (kTasks + NT - 1) / NT;
  u32x4 r[kIters][4];
  __device__ __forceinline__ void load(const __bf16* __restrict__ src, int64_t ld, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * NT;
      const int rq = t % (ROWS / 4), dc = t / (ROWS / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = rq * 4 + j;
        r[it][j] = u32x4{0u, 0u, 0u, 0u};
        if (t < kTasks && row < nvalid) r[it][j] = *reinterpret_cast<const u32x4*>(src + row * ld + dc * 8);
      }
    }
  }
  __device__ __forceinline__ void store(__bf16* __restrict__ dst, int tid) const {
    constexpr int kTP = TPitch<ROWS>::col;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int t = tid + it * NT;
      if (t >= kTasks) continue;
      const int rq = t % (ROWS / 4), dc = t / (ROWS / 4);
      __bf16* base = dst + (dc * 8) * kTP + tslot(rq * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(r[it][1][e >> 1], r[it][0][e >> 1], sel);
        const uint32_t hi = __builtin_amdgcn_perm(r[it][3][e >> 1], r[it][2][e >> 1], sel);
        *reinterpret_cast<u32x2*>(base + e * kTP) = u32x2{lo, hi};
      }
    }
  }
};

// out[dblk] += sum over the 32 contraction rows of block `blk` of
// X[row][d] * vals[i] (vals[i] belongs to row blk*32 + acc_row(i, g)).
// bf16: X is a transposed tile; fp32: X is row-major.
template <typename T, int D, int ROWS>
__device__ __forceinline__ void mma_contract_block(f32x16* out, const T* __restrict__ X, const float* vals,
                                                   int blk, int r32, int g) {
  using M = Mma<T>;
  if constexpr (sizeof(T) == 2) {
    constexpr int kTP = TPitch<ROWS>::col;
    bf16x8 b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) b[u][j] = (__bf16)vals[8 * u + j];
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        out[dblk] = M::mma(M::load(X + (dblk * 32 + r32) * kTP + blk * 32 + 16 * u + 8 * g), b[u], out[dblk]);
  } else {
    constexpr int kPitch = Pitch<T, D>::row;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[dblk] = M::mma(X[(blk * 32 + acc_row(i, g)) * kPitch + dblk * 32 + r32], vals[i], out[dblk]);
  }
}

}  // namespace hstu
