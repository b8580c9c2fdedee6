// api_check.cpp -- drives the host runtime of libfd (fd_api.cpp) through its
// C ABI in a build with AddressSanitizer and UndefinedBehaviorSanitizer,
// against host-only kernel stand-ins (kernels_stub.cpp). TEST
// INFRASTRUCTURE ONLY (tests/test_host_sanitizers.py).
//
// Prints one PLAN line per (problem, forced split count) for the test to
// compare with the real library, runs every entry point on valid arguments
// (host buffers stand in for device memory; nothing is launched) and on one
// malformed argument at a time, and exits non-zero on any unexpected status
// or any launch record pointing outside its workspace.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fd.h"

namespace fd_stub {
extern const char* ws_lo;
extern size_t ws_bytes;
extern int partial_launches, combine_launches, bad_records;
extern char static_area[];
}  // namespace fd_stub

static int failures = 0;

static void expect(fd_status got, fd_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d (%s), expected %d\n", what, got, fd_last_error(), want);
    ++failures;
  }
}

static fd_problem problem(int B, int Hq, int Hkv, int D, int L, int page, int kv, int q_len, int out) {
  fd_problem p;
  std::memset(&p, 0, sizeof p);
  p.batch = B;
  p.num_q_heads = Hq;
  p.num_kv_heads = Hkv;
  p.head_dim = D;
  p.max_seq_len = L;
  p.page_size = page;
  p.num_pages = page ? (L + page - 1) / page * B : 0;
  p.kv_dtype = kv;
  p.q_dtype = kv == FD_FP8_E4M3 ? FD_BF16 : kv;
  p.out_dtype = out;
  p.q_len = q_len;
  return p;
}

// One step's host stand-ins for the device buffers of problem p.
struct Step {
  std::vector<char> q, kv, table, lens, out, lse, scales;
  std::vector<int32_t> host_lens;
  std::vector<char> ws_raw;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  fd_kv_layout lay;
  static char* aligned(std::vector<char>& v, size_t bytes, size_t a) {
    v.assign(bytes + a, 0);
    char* p = v.data();
    return p + (a - reinterpret_cast<uintptr_t>(p) % a) % a;
  }
  Step(const fd_problem& p, const fd_plan& plan) {
    const int qlen = p.q_len ? p.q_len : 1;
    const size_t rows = (size_t)p.batch * qlen * p.num_q_heads;
    aligned(q, rows * p.head_dim * (p.kv_dtype == FD_F32 ? 4 : 2), 16);
    const int64_t tokens = p.page_size ? p.page_size : p.max_seq_len;
    lay.stride_token = p.head_dim;
    lay.stride_head = tokens * p.head_dim;
    lay.stride_outer = p.num_kv_heads * lay.stride_head;
    aligned(kv, 64, 16);
    aligned(scales, 2 * 4 * p.num_kv_heads, 16);
    lay.k_scale = lay.v_scale = reinterpret_cast<const float*>(scales.data());
    aligned(table, 4 * (size_t)p.batch * 4096, 16);
    aligned(lens, 4 * (size_t)p.batch, 16);
    host_lens.assign(p.batch, p.max_seq_len);
    aligned(out, rows * p.head_dim * 4, 16);
    aligned(lse, rows * 4, 16);
    ws_bytes = fd_workspace_size(&p, &plan);
    ws = aligned(ws_raw, ws_bytes + 256, 256);
  }
  const void* qp() { return q.data() + (16 - reinterpret_cast<uintptr_t>(q.data()) % 16) % 16; }
  const void* kvp() { return kv.data() + (16 - reinterpret_cast<uintptr_t>(kv.data()) % 16) % 16; }
  const int32_t* tp(const fd_problem& p) {
    return p.page_size ? reinterpret_cast<const int32_t*>(table.data()) : nullptr;
  }
  const int32_t* lp() { return reinterpret_cast<const int32_t*>(lens.data()); }
  void* op() { return out.data() + (16 - reinterpret_cast<uintptr_t>(out.data()) % 16) % 16; }
  float* sp() { return reinterpret_cast<float*>(lse.data()); }
};

static void run_all(const fd_problem& p, const fd_plan& plan) {
  Step s(p, plan);
  const int32_t bts = p.page_size ? 4096 : 0;
  fd_stub::ws_lo = s.ws;
  fd_stub::ws_bytes = s.ws_bytes;
  expect(fd_decode_partial(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), s.host_lens.data(), s.tp(p), bts,
                           0.1f, s.ws, s.ws_bytes, nullptr, nullptr),
         FD_OK, "partial");
  expect(fd_decode_combine(&p, &plan, s.ws, s.ws_bytes, s.op(), s.sp(), nullptr, nullptr), FD_OK, "combine");
  expect(fd_decode(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), s.host_lens.data(), s.tp(p), bts, 0.1f, s.ws,
                   s.ws_bytes, s.op(), s.sp(), nullptr, nullptr),
         FD_OK, "decode");
  if (s.ws_bytes <= FD_STATIC_WORKSPACE_BYTES) {
    fd_stub::ws_lo = fd_stub::static_area;
    fd_stub::ws_bytes = FD_STATIC_WORKSPACE_BYTES;
    expect(fd_decode_static(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), s.host_lens.data(), s.tp(p), bts,
                            0.1f, s.op(), s.sp(), nullptr),
           FD_OK, "static");
    fd_stub::ws_lo = s.ws;
    fd_stub::ws_bytes = s.ws_bytes;
  }
  // One malformed argument at a time: refused before anything is launched.
  const int before = fd_stub::partial_launches + fd_stub::combine_launches;
  expect(fd_decode_partial(&p, &plan, nullptr, s.kvp(), s.kvp(), &s.lay, s.lp(), nullptr, s.tp(p), bts, 0.1f, s.ws,
                           s.ws_bytes, nullptr, nullptr),
         FD_ERR_INVALID_ARG, "null q");
  expect(fd_decode_partial(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), nullptr, s.tp(p), bts, 0.1f,
                           s.ws + 16, s.ws_bytes, nullptr, nullptr),
         FD_ERR_INVALID_ARG, "misaligned workspace");
  expect(fd_decode_partial(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), nullptr, s.tp(p), bts, 0.1f, s.ws,
                           s.ws_bytes - 1, nullptr, nullptr),
         FD_ERR_WORKSPACE_TOO_SMALL, "short workspace");
  fd_kv_layout bad = s.lay;
  bad.stride_token = p.head_dim - 1;
  expect(fd_decode_partial(&p, &plan, s.qp(), s.kvp(), s.kvp(), &bad, s.lp(), nullptr, s.tp(p), bts, 0.1f, s.ws,
                           s.ws_bytes, nullptr, nullptr),
         FD_ERR_INVALID_ARG, "bad stride");
  std::vector<int32_t> lens = s.host_lens;
  lens[p.batch - 1] = p.max_seq_len + 1;
  expect(fd_decode_partial(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), lens.data(), s.tp(p), bts, 0.1f,
                           s.ws, s.ws_bytes, nullptr, nullptr),
         FD_ERR_INVALID_ARG, "length past max_seq_len");
  lens[p.batch - 1] = 0;
  expect(fd_decode(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), lens.data(), s.tp(p), bts, 0.1f, s.ws,
                   s.ws_bytes, s.op(), s.sp(), nullptr, nullptr),
         FD_ERR_EMPTY_SEQUENCE, "empty sequence");
  expect(fd_decode_combine(&p, &plan, s.ws, s.ws_bytes, static_cast<char*>(s.op()) + 4, s.sp(), nullptr, nullptr),
         FD_ERR_INVALID_ARG, "misaligned out");
  expect(fd_decode_static(&p, &plan, s.qp(), s.kvp(), s.kvp(), &s.lay, s.lp(), nullptr, s.tp(p), bts, 0.1f, nullptr,
                          nullptr, nullptr),
         FD_ERR_INVALID_ARG, "static without out");
  fd_plan wrong = plan;
  wrong.path = FD_PATH_AUTO;
  expect(fd_decode_combine(&p, &wrong, s.ws, s.ws_bytes, s.op(), s.sp(), nullptr, nullptr), FD_ERR_INVALID_ARG,
         "unresolved path");
  if (fd_stub::partial_launches + fd_stub::combine_launches != before) {
    std::fprintf(stderr, "FAIL: a refused call launched\n");
    ++failures;
  }
}

int main() {
  const int dtypes[3] = {FD_F32, FD_BF16, FD_FP8_E4M3};
  const int shapes[][6] = {
      // B, Hq, Hkv, D, L, page
      {1, 1, 1, 64, 1000, 0},     {1, 32, 8, 128, 32768, 0}, {4, 32, 32, 128, 131072, 0},
      {16, 32, 8, 128, 65536, 16}, {128, 32, 8, 128, 2048, 0}, {3, 8, 2, 128, 700, 64},
      {5, 16, 2, 64, 333, 256},    {2, 4, 4, 128, 48, 0},
  };
  const int splits[] = {0, 1, 3, 64};
  int n = 0;
  for (const auto& sh : shapes)
    for (int dt : dtypes)
      for (int q_len : {1, 3}) {
        if (dt == FD_F32 && (sh[2] != sh[1] || q_len != 1)) continue;
        const int out = dt == FD_F32 ? FD_F32 : FD_BF16;
        const fd_problem p = problem(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], dt, q_len, out);
        for (int S : splits) {
          fd_plan plan;
          std::memset(&plan, 0x5a, sizeof plan);
          const fd_status st = fd_plan_splits(&p, 256, S, &plan);
          const size_t ws = st == FD_OK ? fd_workspace_size(&p, &plan) : 0;
          std::printf("PLAN %d %d %d %d %d %d %d %d %d -> %d %d %d %d %d %d %d %d %d %zu\n", p.batch, p.num_q_heads,
                      p.num_kv_heads, p.head_dim, p.max_seq_len, p.page_size, p.kv_dtype, p.q_len, S, st,
                      st == FD_OK ? plan.num_splits : 0, st == FD_OK ? plan.chunk_len : 0,
                      st == FD_OK ? plan.path : 0, st == FD_OK ? plan.mode : 0, st == FD_OK ? plan.workers : 0,
                      st == FD_OK ? plan.tile : 0, st == FD_OK ? plan.lead_workers : 0,
                      st == FD_OK ? plan.lead_pct : 0, ws);
          if (st == FD_OK && ws < ((size_t)256 << 20)) {
            run_all(p, plan);
            ++n;
          }
        }
      }
  // Malformed problems and plans.
  fd_plan plan;
  fd_problem p = problem(2, 6, 4, 128, 100, 0, FD_BF16, 1, FD_BF16);
  expect(fd_plan_splits(&p, 256, 0, &plan), FD_ERR_INVALID_ARG, "Hq not a multiple of Hkv");
  p = problem(2, 8, 4, 96, 100, 0, FD_BF16, 1, FD_BF16);
  expect(fd_plan_splits(&p, 256, 0, &plan), FD_ERR_UNSUPPORTED, "head_dim 96");
  p = problem(2, 8, 4, 128, 100, 48, FD_BF16, 1, FD_BF16);
  expect(fd_plan_splits(&p, 256, 0, &plan), FD_ERR_UNSUPPORTED, "page size 48");
  p = problem(2, 8, 4, 128, 100, 0, FD_BF16, 17, FD_BF16);
  expect(fd_plan_splits(&p, 256, 0, &plan), FD_ERR_UNSUPPORTED, "q_len 17");
  expect(fd_plan_splits(nullptr, 256, 0, &plan), FD_ERR_INVALID_ARG, "null problem");
  if (fd_workspace_size(nullptr, nullptr) != 0) ++failures;
  if (fd_stub::bad_records) failures += fd_stub::bad_records;
  std::printf("RUNS %d partial=%d combine=%d\n", n, fd_stub::partial_launches, fd_stub::combine_launches);
  if (failures) {
    std::fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  std::printf("api_check: ok\n");
  return 0;
}
