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
  int32_t lead_workers;   // balanced mode: the first lead_workers workers take
  int32_t lead_pct;       //   lead_pct % of another worker's tiles (0: uniform)
  int32_t rows_per_seg;   // query rows one segment (and one balanced-mode record) holds
  int32_t segs_per_seq;   // segments per sequence: Hkv * row tiles per KV head
  int32_t q_len;          // query tokens per sequence
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
  int32_t page_shift;     // paged: log2(page_size)
  int32_t kv_dtype;       // fd_dtype; q is bf16 for an fp8 cache, else kv_dtype
  int32_t paged;
  int32_t path;           // FD_PATH_VALU or FD_PATH_MFMA
  Geometry geo;
  float qscale;           // scale * log2(e): scores are kept in base-2 units
  const float* k_scale;   // fp8: [Hkv] dequantisation scales, else nullptr
  const float* v_scale;
  float* o_part;          // split: [rows][S][D]; balanced: [slots][rows_per_seg][D]
  float* lse_part;        // split: [rows][S];    balanced: [slots][rows_per_seg]
  int32_t* tile_prefix;   // balanced: [B + 1] running tile counts, written by the partial launch
  // Single-launch decode (fd_decode): set `out` to merge in the same launch.
  void* out;              // [B][q_len][Hq][D] out_dtype, or nullptr for the two-launch path
  float* lse_out;         // [B][q_len][Hq] or nullptr
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

// Query rows of one segment for a path, given the q_len * group rows of a KV
// head: MFMA takes the largest divisor <= 16, the VALU kernel 4, 2 or 1 (2 or
// 1 for fp8). A segment's rows are a run of the KV head's rows in
// (token, head-in-group) order.
int rows_per_segment(int path, int kv_dtype, int rows_per_kv_head);

// Keys per wave tile of the partial kernel a path / dtype / head_dim uses.
int kernel_tile(int path, int kv_dtype, int head_dim);

// True if an MFMA kernel is built for this shape (rows: per segment).
bool mfma_supported(int kv_dtype, int head_dim, int rows);

// Resident 64-lane waves per compute unit for the balanced kernel of this
// shape on the current device, or 0 when it cannot be queried.
int resident_waves_per_cu(int path, int kv_dtype, int head_dim, int rows, int paged);

hipError_t launch_partial(const PartialLaunch& a, hipStream_t stream);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream);

// fd_decode_static's workspace: a library-owned device array of this many
// bytes per GPU (FD_STATIC_WORKSPACE_BYTES in fd.h).
constexpr size_t kStaticWorkspaceBytes = FD_STATIC_WORKSPACE_BYTES;

// Device address of that array on the GPU `stream` belongs to (the current
// GPU for the null stream), looked up once per device (hipGetSymbolAddress
// with that device made current for the call) and kept.
hipError_t static_workspace(hipStream_t stream, void** ptr);

}  // namespace fd
