// fd_api.cpp -- the C ABI of libfd: planner, workspace sizing, argument
// checks, cross-stream ordering and kernel launches.
//
// Pages cited (by title and section):
//   [MERGE] www.2kiu.com/news/6053916: "分块数量是一笔成本账" (more chunks buy
//           independent work at the price of partial records, launches and
//           merge cost; short contexts can lose) and its closing paragraphs
//           (the merge waits until every chunk result is visible and the
//           records live until it ends; submission is not completion, so
//           asynchronous devices need dependencies or events; the workspace
//           follows the chunk count; pick the path by batch, context,
//           head_dim and device).
//   [INFRA] "AI Infra：深入理解大模型中的数学与Infra优化", 2.6 "Flash-Decoding 的
//           Split-K" (a batch x heads grid alone idles compute units when the
//           query length is one).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fd.h"
#include "fd_internal.h"

namespace {

thread_local std::string g_last_error;

fd_status fail(fd_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr int32_t kChunkQuantum = 16;     // chunk_len granularity: one 16-key group
constexpr int32_t kMinChunk = 256;        // shortest chunk the planner makes on its own
constexpr int kDefaultWavesPerCu = 8;     // resident waves per CU when the device is not asked
constexpr int64_t kInFlightPerCu = 128 << 10;   // K/V bytes in flight per CU the balanced plan aims for
// Leading workers' share of tiles relative to the others, in percent (plan
// bounds, and the planner's choice for kernels that run two worker waves per
// SIMD; see fd_plan_splits).
constexpr int kLeadPctMin = 50, kLeadPctMax = 200, kLeadPctTwoPerSimd = 130;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dtype_ok(int32_t d) { return d == FD_F32 || d == FD_BF16 || d == FD_FP8_E4M3; }

constexpr int32_t kMaxQLen = 16;

// Query tokens per sequence; 0 is read as 1.
int q_len_of(const fd_problem* p) { return p->q_len == 0 ? 1 : p->q_len; }

// Query rows that read one KV head: q_len tokens x the group.
int rows_per_kv_head(const fd_problem* p) { return q_len_of(p) * (p->num_q_heads / p->num_kv_heads); }

fd_status check_problem(const fd_problem* p) {
  if (!p) return fail(FD_ERR_INVALID_ARG, "problem is NULL");
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->max_seq_len < 1)
    return fail(FD_ERR_INVALID_ARG, "batch, heads and max_seq_len must be >= 1");
  if (p->batch > 65535) return fail(FD_ERR_INVALID_ARG, "batch must be <= 65535");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(FD_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(FD_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!dtype_ok(p->q_dtype) || !dtype_ok(p->kv_dtype) || !dtype_ok(p->out_dtype))
    return fail(FD_ERR_INVALID_ARG, "unknown dtype code");
  const bool f32 = p->q_dtype == FD_F32 && p->kv_dtype == FD_F32 && p->out_dtype == FD_F32;
  const bool bf16 = p->q_dtype == FD_BF16 && (p->kv_dtype == FD_BF16 || p->kv_dtype == FD_FP8_E4M3) &&
                    p->out_dtype != FD_FP8_E4M3;
  if (!f32 && !bf16)
    return fail(FD_ERR_UNSUPPORTED,
                "dtypes (q/kv/out) must be f32/f32/f32, bf16/bf16/{bf16,f32} or bf16/fp8/{bf16,f32}");
  if (p->q_len < 0 || p->q_len > kMaxQLen) return fail(FD_ERR_UNSUPPORTED, "q_len must be 1..16 (0 means 1)");
  if (p->page_size != 0 && (p->page_size < 16 || p->page_size > 256 || (p->page_size & (p->page_size - 1))))
    return fail(FD_ERR_UNSUPPORTED, "page_size must be 0 or a power of two from 16 to 256");
  if (p->page_size && p->num_pages < 1) return fail(FD_ERR_INVALID_ARG, "paged cache needs num_pages >= 1");
  if ((int64_t)p->num_kv_heads * rows_per_kv_head(p) > 65535) return fail(FD_ERR_INVALID_ARG, "too many heads");
  return FD_OK;
}

// Query rows a segment (and a balanced-mode record) holds, and segments per
// sequence.
int rows_per_seg(const fd_problem* p, int32_t path) {
  return fd::rows_per_segment(path, p->kv_dtype, rows_per_kv_head(p));
}
int segs_per_seq(const fd_problem* p, int32_t path) {
  return p->num_kv_heads * (rows_per_kv_head(p) / rows_per_seg(p, path));
}

// Balanced mode needs the tile count of the whole batch and the record slots
// to fit 32-bit indices.
bool balanced_fits(const fd_problem* p, int32_t path, int64_t workers) {
  const int64_t tile = fd::kernel_tile(path, p->kv_dtype, p->head_dim);
  const int64_t segs = (int64_t)p->batch * segs_per_seq(p, path);
  const int64_t tiles = segs * ceil_div(p->max_seq_len, tile);
  const int64_t slots = segs + workers - 1;
  return tiles < ((int64_t)1 << 31) && slots * rows_per_seg(p, path) * p->head_dim < ((int64_t)1 << 31);
}

fd_status check_plan(const fd_problem* p, const fd_plan* plan) {
  if (!plan) return fail(FD_ERR_INVALID_ARG, "plan is NULL");
  if (plan->path != FD_PATH_VALU && plan->path != FD_PATH_MFMA)
    return fail(FD_ERR_INVALID_ARG, "plan path must be VALU or MFMA (fd_plan_splits resolves AUTO)");
  if (plan->path == FD_PATH_MFMA && !fd::mfma_supported(p->kv_dtype, p->head_dim, rows_per_seg(p, plan->path)))
    return fail(FD_ERR_UNSUPPORTED,
                "MFMA path needs a bf16 or fp8 cache, head_dim 128 and 4 .. 16 query rows per segment");
  if (plan->mode == FD_MODE_SPLITS) {
    if (plan->num_splits < 1 || plan->chunk_len < kChunkQuantum || plan->chunk_len % kChunkQuantum)
      return fail(FD_ERR_INVALID_ARG, "plan needs num_splits >= 1 and chunk_len a positive multiple of 16");
    if ((int64_t)plan->num_splits * plan->chunk_len < p->max_seq_len)
      return fail(FD_ERR_INVALID_ARG, "plan does not cover max_seq_len");
    if ((int64_t)plan->num_splits * plan->chunk_len > (int64_t)INT32_MAX)
      return fail(FD_ERR_INVALID_ARG, "plan covers more than 2^31 keys");
    if (plan->lead_workers != 0 || plan->lead_pct != 0)
      return fail(FD_ERR_INVALID_ARG, "lead_workers and lead_pct are balanced-mode fields; set them to 0");
    return FD_OK;
  }
  if (plan->mode == FD_MODE_BALANCED) {
    if (plan->workers < 1) return fail(FD_ERR_INVALID_ARG, "balanced plan needs workers >= 1");
    if (plan->tile != fd::kernel_tile(plan->path, p->kv_dtype, p->head_dim))
      return fail(FD_ERR_INVALID_ARG, "balanced plan tile does not match the kernel");
    if (!balanced_fits(p, plan->path, plan->workers))
      return fail(FD_ERR_UNSUPPORTED, "problem too large for balanced mode; use forced splits");
    if (plan->lead_workers < 0 || plan->lead_workers > plan->workers ||
        (plan->lead_pct != 0 && (plan->lead_pct < kLeadPctMin || plan->lead_pct > kLeadPctMax)))
      return fail(FD_ERR_INVALID_ARG, "lead_workers must be in [0, workers] and lead_pct 0 or in [50, 200]");
    return FD_OK;
  }
  return fail(FD_ERR_INVALID_ARG, "unknown plan mode");
}

int32_t choose_path(const fd_problem* p) {
  return fd::mfma_supported(p->kv_dtype, p->head_dim, rows_per_seg(p, FD_PATH_MFMA)) ? FD_PATH_MFMA : FD_PATH_VALU;
}

// Segments of the whole batch: (sequence, KV head, row tile) triples; one
// workgroup each per split in split mode.
int64_t units_per_split(const fd_problem* p, int32_t path) { return (int64_t)p->batch * segs_per_seq(p, path); }

// Workspace sections, in order: the single launch's piece counters (first,
// at a place that depends on the problem and path only, so that the
// two-launch step never writes them under any plan), the records' outputs
// and LSEs, and in balanced mode the running tile counts.
struct Layout {
  size_t counter_bytes, o_off, o_bytes, lse_off, lse_bytes, prefix_off, prefix_bytes, total;
};

Layout layout_of(const fd_problem* p, const fd_plan* plan) {
  Layout l{};
  size_t records;   // query-row records
  if (plan->mode == FD_MODE_SPLITS) {
    records = (size_t)p->batch * q_len_of(p) * p->num_q_heads * plan->num_splits;
    l.prefix_bytes = 0;
  } else {
    const size_t slots = (size_t)p->batch * segs_per_seq(p, plan->path) + plan->workers - 1;
    records = slots * rows_per_seg(p, plan->path);
    l.prefix_bytes = ((size_t)p->batch + 1) * sizeof(int32_t);
  }
  l.counter_bytes = (size_t)p->batch * segs_per_seq(p, plan->path) * sizeof(int32_t);
  l.o_off = align_up(l.counter_bytes, kAlign);
  l.o_bytes = records * p->head_dim * sizeof(float);
  l.lse_off = l.o_off + align_up(l.o_bytes, kAlign);
  l.lse_bytes = records * sizeof(float);
  l.prefix_off = l.lse_off + align_up(l.lse_bytes, kAlign);
  l.total = l.prefix_off + align_up(l.prefix_bytes, kAlign);
  return l;
}

fd::Geometry geometry_of(const fd_problem* p, const fd_plan* plan) {
  fd::Geometry g{};
  g.mode = plan->mode;
  g.num_splits = plan->num_splits;
  g.chunk_len = plan->chunk_len;
  g.workers = plan->workers;
  g.tile = plan->tile;
  g.lead_workers = plan->lead_pct != 0 ? plan->lead_workers : 0;
  g.lead_pct = plan->lead_pct;
  g.rows_per_seg = rows_per_seg(p, plan->path);
  g.segs_per_seq = segs_per_seq(p, plan->path);
  g.q_len = q_len_of(p);
  return g;
}

// One event per device for cross-stream edges. hipStreamWaitEvent captures
// the event's state at the time of the call, so a single event can be
// re-recorded for every edge.
std::mutex g_event_mu;
std::vector<hipEvent_t> g_events;

fd_status order_after(hipStream_t stream, hipStream_t producer) {
  if (!producer || producer == stream) return FD_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FD_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_event_mu);
  if ((int)g_events.size() <= dev) g_events.resize(dev + 1, nullptr);
  if (!g_events[dev]) {
    hipError_t e = hipEventCreateWithFlags(&g_events[dev], hipEventDisableTiming);
    if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
  }
  hipError_t e = hipEventRecord(g_events[dev], producer);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, g_events[dev], 0);
  if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("cross-stream edge: ") + hipGetErrorString(e));
  return FD_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

void log_plan(const char* what, const fd_problem* p, const fd_plan* plan) {
  static const bool on = [] {
    const char* s = std::getenv("FD_LOG");
    return s && *s && std::strcmp(s, "0") != 0;
  }();
  if (on)
    std::fprintf(stderr, "[fd] %s B=%d q_len=%d Hq=%d Hkv=%d D=%d Lmax=%d page=%d kv=%d mode=%s splits=%d chunk=%d "
                 "workers=%d tile=%d lead=%d@%d%% rows=%d path=%s\n", what, p->batch, q_len_of(p),
                 p->num_q_heads, p->num_kv_heads, p->head_dim, p->max_seq_len, p->page_size, p->kv_dtype,
                 plan->mode == FD_MODE_BALANCED ? "balanced" : "splits", plan->num_splits, plan->chunk_len,
                 plan->workers, plan->tile, plan->lead_workers, plan->lead_pct, rows_per_seg(p, plan->path),
                 plan->path == FD_PATH_MFMA ? "mfma" : "valu");
}

}  // namespace

extern "C" {

const char* fd_status_string(fd_status s) {
  switch (s) {
    case FD_OK: return "ok";
    case FD_ERR_INVALID_ARG: return "invalid argument";
    case FD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case FD_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FD_ERR_EMPTY_SEQUENCE: return "empty sequence (seq_len 0)";
    case FD_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fd_last_error(void) { return g_last_error.c_str(); }

fd_status fd_plan_splits(const fd_problem* p, int32_t num_cus, int32_t forced_splits, fd_plan* out) {
  g_last_error.clear();
  fd_status st = check_problem(p);
  if (st != FD_OK) return st;
  if (!out) return fail(FD_ERR_INVALID_ARG, "out is NULL");
  if (forced_splits < 0) return fail(FD_ERR_INVALID_ARG, "forced_splits must be >= 0");
  fd_plan plan;
  std::memset(&plan, 0, sizeof plan);
  plan.path = choose_path(p);
  const int64_t L = p->max_seq_len;
  if (forced_splits > 0) {
    const int64_t S = forced_splits;
    const int64_t C = ceil_div(ceil_div(L, S), kChunkQuantum) * kChunkQuantum;
    if (S * C > INT32_MAX) return fail(FD_ERR_INVALID_ARG, "split plan too large");
    plan.mode = FD_MODE_SPLITS;
    plan.num_splits = (int32_t)S;
    plan.chunk_len = (int32_t)C;
    *out = plan;
    log_plan("plan", p, &plan);
    return FD_OK;
  }
  int waves_per_cu = kDefaultWavesPerCu;
  if (num_cus <= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0) return fail(FD_ERR_HIP, "could not query the compute-unit count");
    const int w = fd::resident_waves_per_cu(plan.path, p->kv_dtype, p->head_dim, rows_per_seg(p, plan.path),
                                            p->page_size != 0);
    if (w > 0) waves_per_cu = w;
  }
  // Workers per CU: enough that their loads in flight (two tiles of K and V
  // each: the one being used and the next) reach kInFlightPerCu, at most one
  // per resident wave slot -- every further worker only adds pieces, records
  // and merge work (measured on MI355X: 4 per CU at 16-KiB tiles, 8 at
  // 8-KiB ones, beat one per wave slot by 1-6 %). And none with fewer than
  // kMinChunk keys of the longest possible batch: a worker pays one memory
  // round trip before its first tile arrives.
  const int64_t tile = fd::kernel_tile(plan.path, p->kv_dtype, p->head_dim);
  const int64_t esz = p->kv_dtype == FD_F32 ? 4 : p->kv_dtype == FD_BF16 ? 2 : 1;
  const int64_t tile_bytes = 2 * tile * p->head_dim * esz;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(waves_per_cu, ceil_div(kInFlightPerCu, 2 * tile_bytes)));
  const int64_t segs = units_per_split(p, plan.path);
  const int64_t max_tiles = segs * ceil_div(L, tile);
  const int64_t min_run = std::max<int64_t>(1, kMinChunk / tile);
  const int64_t workers = std::max<int64_t>(1, std::min<int64_t>(per_cu * num_cus, ceil_div(max_tiles, min_run)));
  if (!balanced_fits(p, plan.path, workers))
    return fail(FD_ERR_UNSUPPORTED, "problem too large for balanced mode; pass forced_splits");
  plan.mode = FD_MODE_BALANCED;
  plan.workers = (int32_t)workers;
  plan.tile = (int32_t)tile;
  // Two worker waves per SIMD (the first num_cus workgroups are dispatched
  // one per CU before the second ones): the older wave of each SIMD wins most
  // issue slots; with even shares it finished ~20 % before its sibling on
  // MI355X (fp8 paged decode). The first half of the workers (workgroups
  // 0 .. num_cus - 1) take a larger share: 130 % measured best of 110-150 %,
  // 3.5 % off the step.
  if (per_cu >= 8 && workers == per_cu * num_cus) {
    plan.lead_workers = (int32_t)(workers / 2);
    plan.lead_pct = kLeadPctTwoPerSimd;
  }
  *out = plan;
  log_plan("plan", p, &plan);
  return FD_OK;
}

size_t fd_workspace_size(const fd_problem* p, const fd_plan* plan) {
  if (check_problem(p) != FD_OK || check_plan(p, plan) != FD_OK) return 0;
  return layout_of(p, plan).total;
}

namespace {

// Checks of a step's arguments other than the workspace, shared by every
// entry point that launches the partial kernel.
fd_status check_step(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                     const fd_kv_layout* kv, const int32_t* seq_lens, const int32_t* seq_lens_host,
                     const int32_t* block_table, int32_t block_table_stride, float scale) {
  fd_status st = check_problem(p);
  if (st != FD_OK) return st;
  if ((st = check_plan(p, plan)) != FD_OK) return st;
  if (!q || !k || !v || !kv || !seq_lens)
    return fail(FD_ERR_INVALID_ARG, "q, k, v, kv layout and seq_lens must be non-NULL");
  if ((p->page_size == 0) != (block_table == nullptr))
    return fail(FD_ERR_INVALID_ARG, "block_table must be given exactly when page_size > 0");
  if (p->page_size && block_table_stride < (int32_t)ceil_div(p->max_seq_len, p->page_size))
    return fail(FD_ERR_INVALID_ARG, "block_table_stride is shorter than max_seq_len needs");
  const size_t esz = p->kv_dtype == FD_F32 ? 4 : p->kv_dtype == FD_BF16 ? 2 : 1;
  const int64_t epl = 16 / (int64_t)esz;
  if (p->kv_dtype == FD_FP8_E4M3 && (!kv->k_scale || !kv->v_scale))
    return fail(FD_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(FD_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  if (kv->stride_outer < 0 || kv->stride_head < 0 || kv->stride_token < p->head_dim ||
      kv->stride_outer % epl || kv->stride_head % epl || kv->stride_token % epl)
    return fail(FD_ERR_INVALID_ARG, "KV strides must be non-negative multiples of 16 bytes, token stride >= D");
  if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale must be finite");
  // Buffer-load offsets are 32-bit and stay inside a 16-key group.
  if (kv->stride_token * (int64_t)esz * 32 >= ((int64_t)1 << 31))
    return fail(FD_ERR_UNSUPPORTED, "token stride too large");
  if (seq_lens_host) {
    for (int b = 0; b < p->batch; ++b) {
      if (seq_lens_host[b] < 0 || seq_lens_host[b] > p->max_seq_len)
        return fail(FD_ERR_INVALID_ARG, "seq_len " + std::to_string(b) + " outside [0, max_seq_len]");
      if (seq_lens_host[b] < q_len_of(p))
        return fail(FD_ERR_EMPTY_SEQUENCE, "seq_len " + std::to_string(b) + " is below q_len: a query sees no key");
    }
  }
  return FD_OK;
}

// A caller's workspace: present, aligned and large enough for the plan.
fd_status check_workspace(const fd_problem* p, const fd_plan* plan, const void* workspace, size_t workspace_bytes) {
  if (!workspace) return fail(FD_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(workspace, kAlign)) return fail(FD_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = layout_of(p, plan).total;
  if (workspace_bytes < need)
    return fail(FD_ERR_WORKSPACE_TOO_SMALL, "workspace needs " + std::to_string(need) + " bytes");
  return FD_OK;
}

// The partial kernel's launch record for checked arguments.
void fill_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                  const fd_kv_layout* kv, const int32_t* seq_lens, const int32_t* block_table,
                  int32_t block_table_stride, float scale, void* workspace, fd::PartialLaunch* a) {
  const Layout lay = layout_of(p, plan);
  std::memset(a, 0, sizeof *a);
  a->q = q;
  a->k = k;
  a->v = v;
  a->seq_lens = seq_lens;
  a->block_table = block_table;
  a->stride_outer = kv->stride_outer;
  a->stride_head = kv->stride_head;
  a->stride_token = kv->stride_token;
  a->block_table_stride = block_table_stride;
  a->batch = p->batch;
  a->num_q_heads = p->num_q_heads;
  a->num_kv_heads = p->num_kv_heads;
  a->head_dim = p->head_dim;
  a->max_seq_len = p->max_seq_len;
  a->num_pages = p->num_pages;
  a->kv_dtype = p->kv_dtype;
  a->paged = p->page_size != 0;
  a->page_shift = 0;
  for (int ps = p->page_size; ps > 1; ps >>= 1) ++a->page_shift;
  a->path = plan->path;
  a->geo = geometry_of(p, plan);
  a->qscale = (float)((double)scale * 1.4426950408889634074);
  a->k_scale = p->kv_dtype == FD_FP8_E4M3 ? kv->k_scale : nullptr;
  a->v_scale = p->kv_dtype == FD_FP8_E4M3 ? kv->v_scale : nullptr;
  char* ws = static_cast<char*>(workspace);
  a->counters = reinterpret_cast<int32_t*>(ws);
  a->o_part = reinterpret_cast<float*>(ws + lay.o_off);
  a->lse_part = reinterpret_cast<float*>(ws + lay.lse_off);
  a->tile_prefix = reinterpret_cast<int32_t*>(ws + lay.prefix_off);
  a->out = nullptr;
  a->lse_out = nullptr;
  a->out_dtype = p->out_dtype;
}

// Checks shared by fd_decode_partial and fd_decode, then the launch record.
fd_status prepare_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                          const fd_kv_layout* kv, const int32_t* seq_lens, const int32_t* seq_lens_host,
                          const int32_t* block_table, int32_t block_table_stride, float scale, void* workspace,
                          size_t workspace_bytes, fd::PartialLaunch* a) {
  fd_status st = check_step(p, plan, q, k, v, kv, seq_lens, seq_lens_host, block_table, block_table_stride, scale);
  if (st != FD_OK) return st;
  if ((st = check_workspace(p, plan, workspace, workspace_bytes)) != FD_OK) return st;
  fill_partial(p, plan, q, k, v, kv, seq_lens, block_table, block_table_stride, scale, workspace, a);
  return FD_OK;
}

// The combine kernel's launch record for checked arguments.
void fill_combine(const fd_problem* p, const fd_plan* plan, const void* workspace, void* out, float* lse_out,
                  fd::CombineLaunch* a) {
  const Layout lay = layout_of(p, plan);
  const char* ws = static_cast<const char*>(workspace);
  a->o_part = reinterpret_cast<const float*>(ws + lay.o_off);
  a->lse_part = reinterpret_cast<const float*>(ws + lay.lse_off);
  a->tile_prefix = reinterpret_cast<const int32_t*>(ws + lay.prefix_off);
  a->out = out;
  a->lse_out = lse_out;
  a->batch = p->batch;
  a->num_q_heads = p->num_q_heads;
  a->num_kv_heads = p->num_kv_heads;
  a->head_dim = p->head_dim;
  a->out_dtype = p->out_dtype;
  a->geo = geometry_of(p, plan);
}

fd_status check_outputs(const void* out, const float* lse_out) {
  if (!out) return fail(FD_ERR_INVALID_ARG, "out must be non-NULL");
  if (!aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return fail(FD_ERR_INVALID_ARG, "out must be 16-byte aligned and lse_out 4-byte aligned");
  return FD_OK;
}

}  // namespace

fd_status fd_decode_partial(const fd_problem* p, const fd_plan* plan, const void* q, const void* k,
                            const void* v, const fd_kv_layout* kv, const int32_t* seq_lens,
                            const int32_t* seq_lens_host, const int32_t* block_table,
                            int32_t block_table_stride, float scale, void* workspace, size_t workspace_bytes,
                            fd_stream stream, fd_stream after_stream) {
  g_last_error.clear();
  fd::PartialLaunch a;
  fd_status st = prepare_partial(p, plan, q, k, v, kv, seq_lens, seq_lens_host, block_table, block_table_stride,
                                 scale, workspace, workspace_bytes, &a);
  if (st != FD_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = order_after(s, reinterpret_cast<hipStream_t>(after_stream))) != FD_OK) return st;
  log_plan("partial", p, plan);
  hipError_t e = fd::launch_partial(a, s);
  if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("partial launch: ") + hipGetErrorString(e));
  return FD_OK;
}

fd_status fd_decode(const fd_problem* p, const fd_plan* plan, const void* q, const void* k, const void* v,
                    const fd_kv_layout* kv, const int32_t* seq_lens, const int32_t* seq_lens_host,
                    const int32_t* block_table, int32_t block_table_stride, float scale, void* workspace,
                    size_t workspace_bytes, void* out, float* lse_out, fd_stream stream, fd_stream after_stream) {
  g_last_error.clear();
  fd::PartialLaunch a;
  fd_status st = prepare_partial(p, plan, q, k, v, kv, seq_lens, seq_lens_host, block_table, block_table_stride,
                                 scale, workspace, workspace_bytes, &a);
  if (st != FD_OK) return st;
  if ((st = check_outputs(out, lse_out)) != FD_OK) return st;
  // The in-kernel merge addresses a segment's records with 32-bit byte offsets.
  const int64_t span = plan->mode == FD_MODE_SPLITS
                           ? (int64_t)q_len_of(p) * p->num_q_heads * plan->num_splits * p->head_dim * 4
                           : ((int64_t)p->batch * segs_per_seq(p, plan->path) + plan->workers) *
                                 rows_per_seg(p, plan->path) * p->head_dim * 4;
  if (span >= ((int64_t)1 << 31))
    return fail(FD_ERR_UNSUPPORTED, "workspace too large for the single-launch merge; use partial + combine");
  a.out = out;
  a.lse_out = lse_out;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = order_after(s, reinterpret_cast<hipStream_t>(after_stream))) != FD_OK) return st;
  log_plan("decode", p, plan);
  hipError_t e = fd::launch_partial(a, s);
  if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  return FD_OK;
}

fd_status fd_decode_combine(const fd_problem* p, const fd_plan* plan, const void* workspace,
                            size_t workspace_bytes, void* out, float* lse_out, fd_stream stream,
                            fd_stream partial_stream) {
  g_last_error.clear();
  fd_status st = check_problem(p);
  if (st != FD_OK) return st;
  if ((st = check_plan(p, plan)) != FD_OK) return st;
  if ((st = check_workspace(p, plan, workspace, workspace_bytes)) != FD_OK) return st;
  if ((st = check_outputs(out, lse_out)) != FD_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = order_after(s, reinterpret_cast<hipStream_t>(partial_stream))) != FD_OK) return st;
  fd::CombineLaunch a;
  fill_combine(p, plan, workspace, out, lse_out, &a);
  hipError_t e = fd::launch_combine(a, s);
  if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("combine launch: ") + hipGetErrorString(e));
  return FD_OK;
}

fd_status fd_decode_static(const fd_problem* p, const fd_plan* plan, const void* q, const void* k,
                           const void* v, const fd_kv_layout* kv, const int32_t* seq_lens,
                           const int32_t* seq_lens_host, const int32_t* block_table, int32_t block_table_stride,
                           float scale, void* out, float* lse_out, fd_stream stream) {
  g_last_error.clear();
  fd_status st = check_step(p, plan, q, k, v, kv, seq_lens, seq_lens_host, block_table, block_table_stride, scale);
  if (st != FD_OK) return st;
  if ((st = check_outputs(out, lse_out)) != FD_OK) return st;
  const size_t need = layout_of(p, plan).total;
  if (need > fd::kStaticWorkspaceBytes)
    return fail(FD_ERR_WORKSPACE_TOO_SMALL, "plan needs " + std::to_string(need) +
                                                " bytes of workspace; the static workspace holds " +
                                                std::to_string(fd::kStaticWorkspaceBytes));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;   // the array of the stream's GPU
  hipError_t e = fd::static_workspace(s, &ws);
  if (e != hipSuccess) return fail(FD_ERR_HIP, std::string("static workspace: ") + hipGetErrorString(e));
  fd::PartialLaunch a;
  fill_partial(p, plan, q, k, v, kv, seq_lens, block_table, block_table_stride, scale, ws, &a);
  log_plan("static", p, plan);
  if ((e = fd::launch_partial(a, s)) != hipSuccess)
    return fail(FD_ERR_HIP, std::string("partial launch: ") + hipGetErrorString(e));
  fd::CombineLaunch c;
  fill_combine(p, plan, ws, out, lse_out, &c);
  if ((e = fd::launch_combine(c, s)) != hipSuccess)
    return fail(FD_ERR_HIP, std::string("combine launch: ") + hipGetErrorString(e));
  return FD_OK;
}

}  // extern "C"
