// Internal declarations shared by the host runtime and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

// Geometry both launches of one plan agree on.
struct Geometry {
  int32_t mode;           // FD_MODE_SPLITS or FD_MODE_BALANCED
  int32_t num_splits;     // split mode: chunks per sequence
  int32_t chunk_len;      // split mode: keys per chunk
  int32_t workers;        // balanced mode: worker waves
  int32_t tile;           // balanced mode: keys per tile of the worker loop
  int32_t heads_per_seg;  // balanced mode: query heads one record holds
  int32_t segs_per_seq;   // balanced mode: records segments per sequence (Hkv * head tiles)
};

// Everything one partial launch needs, already validated by the host code.
struct PartialLaunch {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int64_t stride_outer;   // elements
  int64_t stride_head;
  int64_t stride_token;
  int32_t block_table_stride;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_seq_len;
  int32_t num_pages;
  int32_t kv_dtype;       // fd_dtype; q has the same type
  int32_t paged;
  int32_t path;           // FD_PATH_VALU or FD_PATH_MFMA
  Geometry geo;
  float qscale;           // scale * log2(e): scores are kept in base-2 units
  float* o_part;          // split: [B][Hq][S][D]; balanced: [slots][heads_per_seg][D]
  float* lse_part;        // split: [B][Hq][S];    balanced: [slots][heads_per_seg]
  int32_t* tile_prefix;   // balanced: [B + 1] running tile counts, written by the partial launch
  // Single-launch decode (fd_decode): set `out` to merge in the same launch.
  void* out;              // [B][Hq][D] out_dtype, or nullptr for the two-launch path
  float* lse_out;         // [B][Hq] or nullptr
  int32_t* counters;      // [B * segs_per_seq] pieces finished per segment; zero between launches
  int32_t out_dtype;
};

struct CombineLaunch {
  const float* o_part;
  const float* lse_part;
  const int32_t* tile_prefix;
  void* out;
  float* lse_out;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t out_dtype;
  Geometry geo;
};

// Query-head tile of the VALU kernel for a group size g (1, 2 or 4 heads per
// workgroup; the grid's y axis walks kv_head * (g / tile) + tile index).
int valu_head_tile(int group);

// Keys per wave tile of the partial kernel a path / dtype / head_dim uses.
int kernel_tile(int path, int kv_dtype, int head_dim);

// True if an MFMA kernel is built for this shape.
bool mfma_supported(int kv_dtype, int head_dim, int group);

// Resident 64-lane waves per compute unit for the balanced kernel of this
// shape on the current device, or 0 when it cannot be queried.
int resident_waves_per_cu(int path, int kv_dtype, int head_dim, int group, int paged);

hipError_t launch_partial(const PartialLaunch& a, hipStream_t stream);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream);

}  // namespace fd
