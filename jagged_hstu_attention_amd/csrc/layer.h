// Launchers of the HSTU layer-step kernels (internal interface between the
// host library and the device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace hstu {

struct ProjParams {
  const void* x;    // [T, Dm] bf16
  const void* w;    // [N, Dm] bf16
  void* out[4];     // U, V, Q, K: [T, width[i]] bf16 each
  int width[4];     // H d_v, H d_v, H d_qk, H d_qk (multiples of the tile width)
  int64_t T;
  int64_t Dm;       // multiple of the contraction step
  int64_t N;        // sum of the widths
};

int proj_tile_rows();
int proj_tile_cols();
int proj_tile_k();
int norm_max_width();
int64_t proj_workgroups(int64_t T, int64_t N);  // the projection launch's grid

hipError_t launch_proj(const ProjParams& p, hipStream_t s);
hipError_t launch_norm_gate(const void* o, const void* u, void* y, int64_t T, int width, float eps, hipStream_t s);

}  // namespace hstu
