// Launchers of the Stochastic Length kernels (internal interface between the
// host library and the device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// Kept lengths and their exclusive scan into out_offsets [B+1], then the
// input row of every output row into out_index (token_keys NULL: recency).
hipError_t launch_sl_select(const int64_t* offsets, int64_t B, double alpha, const float* seq_uniform,
                            const uint32_t* token_keys, int64_t* out_offsets, int64_t* out_index, hipStream_t s);

// out[i] = in[index[i]] for i < min(*count, max_rows), rows of row_bytes
// copied as vec_bytes-wide vectors (vec_bytes divides row_bytes and both
// pointers' alignment).
hipError_t launch_gather_rows(const void* in, void* out, int64_t row_bytes, const int64_t* index,
                              const int64_t* count, int64_t max_rows, int vec_bytes, int cus, hipStream_t s);

}  // namespace hstu
