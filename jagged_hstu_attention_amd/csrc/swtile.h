// Swizzled row-major LDS tiles filled with gfx950 direct-to-LDS loads.
//
// A tile holds ROWS rows of D elements as 16-byte chunks with no padding.
// Chunk c of row r lives at slot s(r, c): with lin = r*C + c (C chunks per
// row) and the 256-byte group G = lin / 16, s = 16*G + ((lin % 16) XOR f(G)).
// f is chosen so that both read patterns the kernels use are free of LDS bank
// conflicts on 64 banks:
//   - row reads: 16 lanes read 16 consecutive rows at one chunk (an MFMA
//     operand whose contraction runs along the row);
//   - transpose reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows
//     x 4 consecutive chunks (an MFMA operand contracted over rows).
// A direct-to-LDS load instruction writes 64 lanes x 16 bytes to 64
// consecutive slots, so each lane loads, from global memory, the chunk whose
// swizzled slot is its own.  Rows past `nvalid` are loaded from the last valid
// row instead (callers mask those rows out of every product).
#pragma once

#include "common.h"

namespace hstu {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T, int D> struct SwTile {
  static constexpr int kElems = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int C = D / kElems;                // chunks per row
  static_assert(C >= 4 && (C & (C - 1)) == 0, "chunks per row");

  __device__ static __forceinline__ int f(int G) {
    if constexpr (C >= 16) return ((G & 3) << 2) | ((G >> 2) & 3);
    else if constexpr (C == 8) return ((G & 1) << 2) | ((G >> 1) & 3);
    else return G & 3;
  }
  __device__ static __forceinline__ int slot(int row, int c) {
    const int lin = row * C + c, G = lin >> 4;
    return (G << 4) | ((lin & 15) ^ f(G));
  }
  // Element offset of (row, element e) in the tile.
  __device__ static __forceinline__ int off(int row, int e) {
    return slot(row, e / kElems) * kElems + (e % kElems);
  }
};

// Byte offset, from a tile's first row in global memory, of the chunk that
// lane `tid` loads in its wave's first direct-to-LDS instruction.  The wave's
// later instructions (every NT/64-th) fill slots NT further on: rows NT/C
// further down with the same chunk order (the swizzle repeats every 16 rows or
// fewer), so one offset per lane serves them all, and all tiles with the same
// row stride.
template <typename T, int D, int NT>
__device__ __forceinline__ uint32_t tile_lane_offset(int tid, int64_t ld) {
  using S = SwTile<T, D>;
  static_assert((NT / 16) % 16 == 0, "the swizzle must repeat between a wave's instructions");
  const int G = tid >> 4;
  const int lin = (G << 4) | ((tid & 15) ^ S::f(G));
  return (uint32_t)((lin / S::C) * ld + (lin % S::C) * S::kElems) * (uint32_t)sizeof(T);
}

// Buffer resource for raw (unstructured) loads from `base`: no stride, the
// whole 32-bit offset range valid, default gfx9 data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
}

// Issue the direct-to-LDS loads of ROWS rows (row r at src + r*ld) into `dst`,
// as buffer loads from a resource based at the tile's first row: the lane's
// 32-bit offset is the only vector operand.  The loads complete asynchronously
// (vmcnt); wait and barrier before reading.  A full tile (nvalid == ROWS) uses
// the offset from tile_lane_offset plus a scalar row shift per instruction; a
// partial tile clamps each row to the last valid one.  The caller must ensure
// ROWS * ld * sizeof(T) < 2^32.  AUX is the loads' cache policy (0: default;
// 2: non-temporal, for data read once).
template <typename T, int D, int ROWS, int NT, int AUX = 0>
__device__ __forceinline__ void tile_load_async(T* __restrict__ dst, const T* __restrict__ src, int64_t ld,
                                                int nvalid, int tid, uint32_t lane_off) {
  using S = SwTile<T, D>;
  using LdsPtr = __attribute__((address_space(3))) void*;
  constexpr int kInstr = ROWS * S::C / 64;
  constexpr int kWaves = NT / 64;
  static_assert(ROWS * S::C % 64 == 0 && kInstr % kWaves == 0, "whole wave instructions");
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS destinations stay scalar
  const __amdgpu_buffer_rsrc_t rs = raw_rsrc(src);
  if (nvalid >= ROWS) {
#pragma unroll
    for (int k = 0; k < kInstr / kWaves; ++k) {
      const uint32_t shift = (uint32_t)(k * (NT / S::C) * ld * (int64_t)sizeof(T));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(dst + (wave + k * kWaves) * 64 * S::kElems), 16,
                                               lane_off, shift, 0, AUX);
    }
    return;
  }
  const int lane = tid & 63;
#pragma unroll
  for (int i = wave; i < kInstr; i += kWaves) {
    const int s = i * 64 + lane;
    const int G = s >> 4;
    const int lin = (G << 4) | ((s & 15) ^ S::f(G));
    const int row = min(lin / S::C, nvalid - 1);
    const uint32_t off = (uint32_t)(row * ld + (lin % S::C) * S::kElems) * (uint32_t)sizeof(T);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(dst + i * 64 * S::kElems), 16, off, 0, 0, AUX);
  }
}

// Instructions per wave of a full tile's tile_load_async.
template <typename T, int D, int ROWS, int NT>
constexpr int tile_load_steps() {
  return ROWS * SwTile<T, D>::C / 64 / (NT / 64);
}

// Instruction k (0 <= k < tile_load_steps) of this wave's tile_load_async, so
// that a caller can spread a tile's loads between its MFMAs: a direct-to-LDS
// load holds the wave at its issue while the memory pipeline accepts it, and
// the MFMAs issued before it keep the matrix pipe busy meanwhile.  A partial
// tile issues all of its (clamped) loads at k = 0.  Together the steps load
// what tile_load_async loads.
template <typename T, int D, int ROWS, int NT, int AUX = 0>
__device__ __forceinline__ void tile_load_step(T* __restrict__ dst, const T* __restrict__ src, int64_t ld,
                                               int nvalid, int tid, uint32_t lane_off, int k) {
  using S = SwTile<T, D>;
  using LdsPtr = __attribute__((address_space(3))) void*;
  constexpr int kWaves = NT / 64;
  if (nvalid >= ROWS) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t shift = (uint32_t)(k * (NT / S::C) * ld * (int64_t)sizeof(T));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(src), (LdsPtr)(dst + (wave + k * kWaves) * 64 * S::kElems), 16,
                                             lane_off, shift, 0, AUX);
  } else if (k == 0) {
    tile_load_async<T, D, ROWS, NT, AUX>(dst, src, ld, nvalid, tid, lane_off);
  }
}

// Wait for every outstanding memory operation of this wave (the direct-to-LDS
// loads among them); a barrier afterwards publishes the tile to the workgroup.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0); }

// MFMA operand of one lane from a row read: row `row`, contraction slice
// starting at element e (kEpl elements).
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::operand tile_row_operand(const T* __restrict__ tile, int row, int e) {
  return Mma<T>::load(tile + SwTile<T, D>::off(row, e));
}

// Four consecutive rows r0..r0+3 of column `col`, via the transpose read: the
// 16 lanes of a lane group cooperate; this lane passes the address of row
// r0 + m/4, columns col0 + 4*(m%4) .. +3 of its group (m = lane % 16) and
// receives column col0 + m.  `row` and `col` are this lane's address
// coordinates (see tr_coords).
template <int D>
__device__ __forceinline__ s16x4 tile_tr4(const __bf16* __restrict__ tile, int row, int col) {
  const __bf16* p = tile + SwTile<__bf16, D>::off(row, col);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Contraction over the 32 rows of block `blk` of a bf16 tile X (rows = the
// contraction index, columns = d):  out[dblk] += X[rows][d]^T-slices * vals,
// with vals[i] the weight of row blk*32 + acc_row(i, g) for this lane's output
// column.  The A operand of MFMA u needs rows 16u + 4g + {0..3} and
// 16u + 8 + 4g + {0..3} of the block at column dblk*32 + r32, i.e. two
// transpose reads.
template <typename T, int D>
__device__ __forceinline__ void tile_contract_block(f32x16* out, const T* __restrict__ X, const float* vals,
                                                    int blk, int lane) {
  using M = Mma<T>;
  const int g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    bf16x8 b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      b[u] = to_bf16x8(vals + 8 * u);
    const int m = lane & 15, q = lane >> 4;
    const int rb = blk * 32 + 4 * g + (m >> 2);
    const int cb = 16 * (q & 1) + 4 * (m & 3);
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const s16x4 lo = tile_tr4<D>(X, rb + 16 * u, dblk * 32 + cb);
        const s16x4 hi = tile_tr4<D>(X, rb + 16 * u + 8, dblk * 32 + cb);
        const short __attribute__((ext_vector_type(8))) a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        out[dblk] = M::mma(__builtin_bit_cast(bf16x8, a), b[u], out[dblk]);
      }
  } else {
    const int r32 = lane & 31;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[dblk] = M::mma(X[SwTile<T, D>::off(blk * 32 + acc_row(i, g), dblk * 32 + r32)], vals[i], out[dblk]);
  }
}

// acc (32 tile-rows x 32 lanes) = sum over d of tile[row][d] * op[d].
template <typename T, int D>
__device__ __forceinline__ f32x16 tile_mma_rows(const T* __restrict__ tile, int row,
                                                const typename Mma<T>::operand* op, int g) {
  using M = Mma<T>;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / M::kK; ++kk)
    acc = M::mma(tile_row_operand<T, D>(tile, row, kk * M::kK + g * M::kEpl), op[kk], acc);
  return acc;
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

// Per-lane byte offsets of the LDS reads one lane makes into a bf16 tile,
// computed once per work item (the swizzle is the same for rows 32 apart and,
// for transpose reads, for rows 16 apart, so block and step offsets are
// compile-time constants added to these).
template <int D> struct LaneOffsets {
  int row[D / 16];     // row reads: row r32, elements kk*16 + 8g
  int tr[D / 32][2];   // transpose reads: rows rb + 8h, columns dblk*32 + cb
  __device__ __forceinline__ void init(int lane) {
    using S = SwTile<__bf16, D>;
    const int r32 = lane & 31, g = lane >> 5, m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = 2 * S::off(r32, kk * 16 + 8 * g);
    const int rb = 4 * g + (m >> 2), cb = 16 * (q & 1) + 4 * (m & 3);
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int h = 0; h < 2; ++h) tr[dblk][h] = 2 * S::off(rb + 8 * h, dblk * 32 + cb);
  }
};

// Same products as tile_mma_rows / tile_contract_block, for bf16 tiles, with
// precomputed lane offsets (`base` is the tile's LDS byte address).
template <int D>
__device__ __forceinline__ f32x16 tile_mma_rows_o(const char* __restrict__ base, const LaneOffsets<D>& lo, int blk,
                                                  const bf16x8* op) {
  using M = Mma<__bf16>;
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    acc = M::mma(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + lo.row[kk] + blk * 32 * D * 2)),
                 op[kk], acc);
  return acc;
}

template <int D>
__device__ __forceinline__ void tile_contract_block_o(f32x16* out, const char* __restrict__ base,
                                                      const LaneOffsets<D>& lo, const float* vals, int blk) {
  using M = Mma<__bf16>;
  bf16x8 b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    b[u] = to_bf16x8(vals + 8 * u);
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* p0 = base + lo.tr[dblk][0] + (blk * 32 + 16 * u) * D * 2;
      const char* p1 = base + lo.tr[dblk][1] + (blk * 32 + 16 * u) * D * 2;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const short __attribute__((ext_vector_type(8))) a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      out[dblk] = M::mma(__builtin_bit_cast(bf16x8, a), b[u], out[dblk]);
    }
}

}  // namespace hstu

namespace hstu {

}  // namespace hstu

namespace hstu {

// Split forms of tile_mma_rows_o / tile_contract_block_o: the LDS reads of a
// product are issued as one group (operands held in registers), so its MFMAs
// run back to back instead of each waiting for its own read.
template <int D>
__device__ __forceinline__ void rows_load(bf16x8* a, const char* __restrict__ base, const LaneOffsets<D>& lo, int blk) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    a[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + lo.row[kk] + blk * 32 * D * 2));
}

template <int D>
__device__ __forceinline__ f32x16 rows_mma(const bf16x8* a, const bf16x8* op) {
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) acc = Mma<__bf16>::mma(a[kk], op[kk], acc);
  return acc;
}

template <int D>
__device__ __forceinline__ void tr_load(bf16x8* t, const char* __restrict__ base, const LaneOffsets<D>& lo, int blk) {
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* p0 = base + lo.tr[dblk][0] + (blk * 32 + 16 * u) * D * 2;
      const char* p1 = base + lo.tr[dblk][1] + (blk * 32 + 16 * u) * D * 2;
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const short __attribute__((ext_vector_type(8))) a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      t[2 * dblk + u] = __builtin_bit_cast(bf16x8, a);
    }
}

template <int D>
__device__ __forceinline__ void tr_mma(f32x16* out, const bf16x8* t, const float* vals) {
  bf16x8 b[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    b[u] = to_bf16x8(vals + 8 * u);
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int u = 0; u < 2; ++u) out[dblk] = Mma<__bf16>::mma(t[2 * dblk + u], b[u], out[dblk]);
}

}  // namespace hstu
