// Device-side building blocks shared by the gfx950 kernels: MFMA operand
// traits, conversions and the work-item format.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxBuckets = 512;

// Work item: one tile of rows of one sequence.  For query tiles `row0` is the
// row in q/out (rank-local when context-parallel), `pos0` the position inside
// the sequence of the first row, `n` the row count, and [w0, w1) the part of
// the tile's walk over 64-key tiles that the item covers (the whole walk
// unless the tile is split); a split tile's part writes fp32 partial sums to
// slot `slot` (-1: not split, the item writes the output itself).  For key
// tiles `row0` is the global row in k/v (w0, w1, slot unused).
struct Item {
  int32_t b;
  int32_t row0;
  int32_t pos0;
  int32_t n;
  int32_t w0;
  int32_t w1;
  int32_t slot;
  int32_t pad;
};

// A query tile whose key walk is split over several items: its rows, and the
// partial-sum slots slot0 .. slot0 + nparts - 1 its parts wrote (in walk
// order).
struct SplitTile {
  int32_t row0;
  int32_t n;
  int32_t slot0;
  int32_t nparts;
};

// Counters written by the scheduler, read by the attention kernels.
enum Ctr : int {
  kCtrQTiles = 0,   // number of query items (tiles or tile parts) in the list
  kCtrQNext = 1,    // work counter popped by the forward / dQ kernel
  kCtrKTiles = 2,   // number of key tiles
  kCtrKNext = 3,    // work counter popped by the dK/dV kernel
  kCtrQNext2 = 4,   // second query-tile counter (backward dQ pass)
  kCtrSplits = 5,   // number of split query tiles
  kCtrGMode = 6,    // 1: the stored score gradient applies to this schedule (every query
                    // segment starts, and ends or meets the sequence end, on a 128-row boundary)
  kCtrCount = 64
};

// ---------------------------------------------------------------------------
// MFMA operand traits.  Both element types use the 32x32 output block, whose
// accumulator layout is: lane l holds column (l % 32), and its 16 values hold
// rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.  An A operand lane (r, g) =
// (l % 32, l / 32) supplies row r and the K slice [g*EPL, (g+1)*EPL) of one
// instruction; a B operand lane supplies column r and the same K slice.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  using operand = bf16x8;
  static constexpr int kK = 16;   // contraction length per instruction
  static constexpr int kEpl = 8;  // operand elements per lane
  __device__ static inline f32x16 mma(operand a, operand b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline operand load(const __bf16* p) {
    return __builtin_bit_cast(operand, *reinterpret_cast<const u32x4*>(p));
  }
};

template <> struct Mma<float> {
  using operand = float;
  static constexpr int kK = 2;
  static constexpr int kEpl = 1;
  __device__ static inline f32x16 mma(operand a, operand b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline operand load(const float* p) { return *p; }
};

// Row (within its 32-row block) of accumulator value i held by lane group g.
__device__ __forceinline__ int acc_row(int i, int g) { return ((i >> 2) << 3) + (g << 2) + (i & 3); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest even) and packed, lo in the low half:
// one v_cvt_pk_bf16_f32 (converting the halves separately and merging them
// takes three instructions).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Eight floats as one bf16 MFMA operand.
__device__ __forceinline__ bf16x8 to_bf16x8(const float* v) {
  const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
  return __builtin_bit_cast(bf16x8, w);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

}  // namespace hstu
