// Parameters and launchers of the attention kernels (internal interface
// between the host library and the device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace hstu {

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const int64_t* offsets;    // [B+1] global
  const int64_t* local_off;  // [B+1] rank-local query offsets
  const int64_t* ts;         // [T]
  const void* w;             // [H, NB]
  void* out;
  void* dq;
  void* dk;
  void* dv;
  float* dw_acc;             // [H, NB] fp32 workspace sums, zeroed by the scheduler, added to by
                             // the dK/dV pass
  float* dw;                 // [H, NB] fp32 output d(ts_weights), written by the dQ pass
  const Item* qitems;
  const Item* kitems;
  int* ctr;
  const uint32_t* edges;     // [NB+1]
  const u32x2* lut;          // [1024] exact-bucket table
  // Candidates (forward only): the last num_targets[b] rows of sequence b
  // attend to the sequence's other rows and to themselves only; with
  // targets_only the query rows are those candidates alone.  NULL: none.
  const int64_t* num_targets;
  int targets_only;
  // Stored score gradients (backward, bf16, d >= 64; NULL: the dQ pass
  // recomputes them).  They are written and read only when the scheduler set
  // ctr[kCtrGMode] (a context-parallel share whose chunk boundaries are not
  // 128-row aligned recomputes them).  G of sequence b, head h is kept in blocks of
  // kGKeys keys x kGRows query rows, block (query tile i, key tile t) at
  // index gblk_off[b] + h n(n+1) + i(i+1) + t with n = ceil(L_b / kGRows)
  // (query tile i sees key tiles 0 .. 2i+1), each block a row-major
  // [kGKeys][kGRows] bf16 tile (key rows, query columns).  Indices >= g_blocks
  // are never touched.
  uint16_t* g;
  const int64_t* gblk_off;  // [B+1]
  int64_t g_blocks;
  // Split query tiles (see Item): the partial sums of part slot s, head h are
  // rows 0 .. n-1 of parts + (s * H + h) * kSplitRows * d, fp32 [rows][d],
  // unscaled accumulators.  NULL when no tile can be split.
  float* parts;
  const SplitTile* splits;  // [split tiles], count in ctr[kCtrSplits]
  int H;
  int NB;
  int cp_size;
  int cp_rank;
  float alpha;
};

// Key-range splitting of query tiles, for problems with too few (tile, head)
// items to fill the chip: the balance target is kQuerySlots workgroups (256
// compute units at two workgroups each, the occupancy of the d = 128 query
// passes), and no part covers fewer than kMinPartTiles 64-key tiles.
constexpr int kQuerySlots = 512;
constexpr int kMinPartTiles = 16;
constexpr int kSplitRows = 128;  // rows of a query tile (partial-sum slot height)

constexpr int kGKeys = 64;    // key rows of a stored-G block
constexpr int kGRows = 128;   // query rows (columns) of a stored-G block
constexpr int kGBlockBytes = kGKeys * kGRows * 2;

// which: 0 forward, 1 dK/dV/dW pass, 2 dQ pass.  max_items bounds the number
// of (tile, head) work items (the grid never exceeds it).
hipError_t launch_attn(const AttnParams& p, bool bf16, int d, int which, int max_items, int cus, hipStream_t s);

// Sum the partial slots of every split query tile (in part order) into the
// output of pass `which` (0: the forward's out, 2: the dQ pass's dq), with
// that pass's output scale.  max_splits bounds the number of split tiles (the
// count itself is read from the counters).
hipError_t launch_reduce(const AttnParams& p, bool bf16, int d, int which, int max_splits, hipStream_t s);

int attn_q_tile_rows();   // query rows per forward / dQ item
int attn_k_tile_keys();   // keys per tile in the forward / dQ loops
int attn_bwd_key_tile(bool bf16, int d);  // keys per dK/dV item
int attn_bwd_q_step();    // query rows per step of the dK/dV loop

// Scheduler: builds the descending-cost tile lists, the rank-local offsets,
// the edge table copy and zero-fills dw.
struct SchedParams {
  const int64_t* offsets;
  int64_t B;
  int cp_size;
  int cp_rank;
  int q_tile;        // rows per query tile (0 = no query list)
  int q_cost_tile;   // key-tile size used in a query tile's cost
  int k_tile;        // keys per key tile (0 = no key list)
  int k_cost_tile;   // query rows per step used in a key tile's cost
  int hist_size;     // cost histogram bins (costs are clamped to hist_size-1)
  int64_t* local_off;
  const int64_t* num_targets;  // as in AttnParams (NULL: none)
  int targets_only;
  int* qtile_off;    // [B+1] first query tile of each sequence in tile order
  int* ktile_off;    // [B+1] first key tile of each sequence
  int64_t* gblk_off; // [B+1] first stored-G block of each sequence (NULL: none)
  int g_heads;       // heads of the stored-G blocks
  int heads;         // heads of the query items (the split balance counts tile x head items)
  int q_extra;       // > 0: long query tiles may be split, into at most q_extra parts beyond
                     // one per tile; 0: never
  SplitTile* splits; // [split tiles] (when q_extra > 0)
  Item* qitems;
  Item* kitems;
  int* ctr;
  uint32_t* edges_out;
  u32x2* lut_out;    // [1024] exact-bucket table
  float* dw;         // zero-filled when non-null
  int dw_count;
  int NB;
};

struct EdgeArg {
  uint32_t e[kMaxBuckets + 1];
};

hipError_t launch_sched(const SchedParams& p, const EdgeArg& edges, hipStream_t s);

constexpr int kSchedHist = 4096;

// Device-side check of the caller's offsets contract (one workgroup).  The
// result is a bit set of CheckBits written to *flag (the flag is cleared by
// the kernel itself first).  total_q < 0 skips the row-count check.
enum CheckBits : int {
  kBadFirst = 1,   // offsets[0] != 0
  kBadOrder = 2,   // offsets decrease somewhere
  kBadTotal = 4,   // offsets[B] != total_kv
  kBadMaxLen = 8,  // a sequence is longer than max_seq_len
  kBadSumSq = 16,  // sum of squared lengths exceeds the stated bound
  kBadRows = 32    // the query rows implied by the offsets differ from total_q
};
struct CheckParams {
  const int64_t* offsets;
  int64_t B;
  int64_t total_kv;
  int64_t max_seq_len;
  int64_t sum_sq_len;  // 0: not checked
  int64_t total_q;     // < 0: not checked
  int cp_size;
  int cp_rank;
  const int64_t* num_targets;  // rows counted are the clamped candidates when targets_only
  int targets_only;
};
hipError_t launch_check(const CheckParams& p, int* flag, hipStream_t s);
// Device address of the library's check flag on the current device (looked up
// once per device).
hipError_t check_flag_ptr(int** out);

hipError_t launch_reorder(const void* in, void* out, int64_t row_bytes, const int64_t* offsets, int64_t B,
                          int64_t total_rows, int64_t max_seq_len, int cp_size, bool inverse,
                          int64_t* out_offsets, hipStream_t s);

}  // namespace hstu
