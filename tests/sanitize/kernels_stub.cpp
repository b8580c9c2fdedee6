// kernels_stub.cpp -- host-only stand-ins for the kernel side of libfd
// (fd_kernels.hip), so that the host runtime (fd_api.cpp) can be built with
// AddressSanitizer and UndefinedBehaviorSanitizer and driven on a machine
// without a GPU. TEST INFRASTRUCTURE ONLY (tests/test_host_sanitizers.py).
//
// The geometry helpers return what the kernels' engines define (rows per
// segment, tile sizes, where the MFMA path is built); the test checks the
// plans this build makes against the real library's. The launchers launch
// nothing: they record the launch and check that every workspace section it
// names lies inside the workspace the host code was given.
#include <cstdio>
#include <cstdlib>

#include "fd_internal.h"

namespace fd_stub {
const char* ws_lo = nullptr;   // the workspace of the call under test
size_t ws_bytes = 0;
int partial_launches = 0, combine_launches = 0, bad_records = 0;
alignas(256) char static_area[fd::kStaticWorkspaceBytes];

void inside(const void* p, size_t bytes, const char* what) {
  const char* c = static_cast<const char*>(p);
  if (!ws_lo || c < ws_lo || c + bytes > ws_lo + ws_bytes) {
    std::fprintf(stderr, "launch record: %s outside the workspace\n", what);
    ++bad_records;
  }
}
}  // namespace fd_stub

namespace fd {

int rows_per_segment(int path, int kv_dtype, int n) {
  if (path == FD_PATH_MFMA) {
    for (int r = 16; r > 1; --r)
      if (n % r == 0) return r;
    return 1;
  }
  if (kv_dtype != FD_FP8_E4M3 && n % 4 == 0) return 4;
  return n % 2 == 0 ? 2 : 1;
}

int kernel_tile(int path, int kv_dtype, int head_dim) {
  if (path == FD_PATH_MFMA) return 32;
  const int esz = kv_dtype == FD_F32 ? 4 : kv_dtype == FD_BF16 ? 2 : 1;
  const int lanes_per_row = head_dim / (16 / esz);   // one 16-byte load per lane
  return 8 * (64 / lanes_per_row);                   // 8 wave loads per tile
}

bool mfma_supported(int kv_dtype, int head_dim, int rows) {
  return (kv_dtype == FD_BF16 || kv_dtype == FD_FP8_E4M3) && head_dim == 128 && rows >= 4 && rows <= 16;
}

int resident_waves_per_cu(int, int, int, int, int) { return 0; }

hipError_t launch_partial(const PartialLaunch& a, hipStream_t) {
  ++fd_stub::partial_launches;
  const Geometry& g = a.geo;
  const size_t records = g.mode == FD_MODE_SPLITS
                             ? (size_t)a.batch * g.q_len * a.num_q_heads * g.num_splits
                             : ((size_t)a.batch * g.segs_per_seq + g.workers - 1) * g.rows_per_seg;
  fd_stub::inside(a.counters, (size_t)a.batch * g.segs_per_seq * 4, "counters");
  fd_stub::inside(a.o_part, records * a.head_dim * 4, "O_part");
  fd_stub::inside(a.lse_part, records * 4, "LSE_part");
  if (g.mode == FD_MODE_BALANCED) fd_stub::inside(a.tile_prefix, ((size_t)a.batch + 1) * 4, "tile counts");
  return hipSuccess;
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t) {
  ++fd_stub::combine_launches;
  const Geometry& g = a.geo;
  const size_t records = g.mode == FD_MODE_SPLITS
                             ? (size_t)a.batch * g.q_len * a.num_q_heads * g.num_splits
                             : ((size_t)a.batch * g.segs_per_seq + g.workers - 1) * g.rows_per_seg;
  fd_stub::inside(a.o_part, records * a.head_dim * 4, "O_part");
  fd_stub::inside(a.lse_part, records * 4, "LSE_part");
  if (g.mode == FD_MODE_BALANCED) fd_stub::inside(a.tile_prefix, ((size_t)a.batch + 1) * 4, "tile counts");
  return hipSuccess;
}

hipError_t static_workspace(hipStream_t, void** ptr) {
  *ptr = fd_stub::static_area;
  return hipSuccess;
}

}  // namespace fd
