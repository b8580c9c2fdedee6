// Internal declarations shared by the host runtime and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

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
  int32_t num_splits;
  int32_t chunk_len;
  int32_t kv_dtype;       // fd_dtype; q has the same type
  int32_t paged;
  int32_t path;           // FD_PATH_VALU or FD_PATH_MFMA
  float qscale;           // scale * log2(e): scores are kept in base-2 units
  float* o_part;          // [B][Hq][S][D]
  float* lse_part;        // [B][Hq][S]
};

struct CombineLaunch {
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse_out;
  int32_t rows;           // B * Hq
  int32_t num_splits;
  int32_t head_dim;
  int32_t out_dtype;
};

// Query-head tile of the VALU kernel for a group size g (1, 2 or 4 heads per
// workgroup; the grid's y axis walks kv_head * (g / tile) + tile index).
int valu_head_tile(int group);

// True if an MFMA kernel is built for this shape.
bool mfma_supported(int kv_dtype, int head_dim, int group);

hipError_t launch_partial(const PartialLaunch& a, hipStream_t stream);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream);

}  // namespace fd
