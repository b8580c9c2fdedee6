/*
 * fd.h -- split-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * One decode step computes, for every sequence b, query token t and query
 * head h, the attention of one query vector over the keys of its KV cache
 * that it may see:
 *
 *     n     = L_b - q_len + 1 + t    (keys 0 .. n-1; n = L_b when q_len = 1)
 *     s_j   = scale * <q[b,t,h], k[b, h/g, j]>          (g = Hq / Hkv), j < n
 *     out   = sum_j exp(s_j - m) v[b, h/g, j] / sum_j exp(s_j - m),  m = max_j s_j
 *     lse   = m + log(sum_j exp(s_j - m))               (natural log)
 *
 * in two launches, as the pages below describe Flash-Decoding:
 *   fd_decode_partial  -- the key range is cut into pieces; every piece writes
 *                         its normalised weighted value sum and its
 *                         log-sum-exp to a workspace.
 *   fd_decode_combine  -- merges the piece records of each output row with
 *                         weights exp(LSE_i - max_i LSE_i).
 * or in one (fd_decode).
 *
 * q_len > 1 is multi-token decode (speculative verification): the q_len
 * query tokens are the sequence's last q_len positions, already in the
 * cache, and token t sees the keys at or before its own position -- the
 * causal rule that [INFRA] 2.5 says a one-token decode step does not need.
 *
 * An fp8 (E4M3) cache holds round(x / scale[kv head]) per element, with one
 * float scale per KV head for K and one for V; the kernels use
 * decode(byte) * scale. [INFRA] 04 lists this KV quantisation among the
 * KV-cache optimisations; E4M3 is the OCP format (bias 7, no infinities,
 * S.1111.111 = NaN).
 *
 * Pages cited (by title and section):
 *   [QA]    "FlashDecoding面经-vivj啥关系 vi就是原来的O呗用LSE是为了防止溢出吗"
 *           (www.gtnt.cn/news/53829), parts 二 (a chunk divides its
 *           accumulator by its local denominator before writing it out) and
 *           三 (LSE_i = m_i + log l_i; merge weights exp(LSE_i - LSE_max)).
 *   [MERGE] www.2kiu.com/news/6053916: "用 log-sum-exp 给块结果定权重"
 *           (chunk output + lse; softmax over lse weighs the chunks; an empty
 *           chunk must not become a zero output with normal weight),
 *           "分块数量是一笔成本账" (cost of the chunk count; masks consistent
 *           across chunks; paged logical order; GQA head mapping), and its
 *           closing paragraphs (workspace lifetime, events, path choice by
 *           batch, context, head_dim and device).
 *   [INFRA] "AI Infra：深入理解大模型中的数学与Infra优化", sections 2.4 (scale),
 *           2.5 (masked keys leave numerator and denominator; decode needs no
 *           causal mask; block-table gather of KV pages), 2.6 (online softmax,
 *           "LSE 与 Online Softmax", "Flash-Decoding 的 Split-K").
 *
 * Conventions for every entry point:
 *   - Every device pointer is caller-owned device memory on the current HIP
 *     device. The library never allocates or frees device memory.
 *   - Nothing throws or aborts across this boundary. Each call returns an
 *     fd_status; fd_last_error() gives a message for the last failure on the
 *     calling thread.
 *   - Argument checks run on the host before any HIP call. A failed check
 *     launches nothing.
 *   - fd_stream is a hipStream_t passed as an opaque pointer (NULL = the
 *     null stream of the current device).
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
  FD_OK = 0,
  FD_ERR_INVALID_ARG = -1,        /* null pointer, bad shape, bad stride, plan mismatch */
  FD_ERR_UNSUPPORTED = -2,        /* head_dim, dtype combination or page size not built */
  FD_ERR_WORKSPACE_TOO_SMALL = -3,
  FD_ERR_EMPTY_SEQUENCE = -4,     /* a host-visible seq_len is 0: no valid key to attend to */
  FD_ERR_HIP = -5                 /* a HIP runtime call or launch failed */
} fd_status;

typedef enum fd_dtype { FD_F32 = 0, FD_BF16 = 1, FD_FP8_E4M3 = 2 } fd_dtype;

/* Which partial kernel runs. FD_PATH_AUTO lets fd_plan_splits choose. */
typedef enum fd_path {
  FD_PATH_AUTO = 0,
  FD_PATH_VALU = 1,   /* vector-ALU dot products: any shape and dtype */
  FD_PATH_MFMA = 2    /* bf16 or fp8 KV, head_dim 128, at least 4 query rows per KV head and tile
                         (q_len * group rows, cut into tiles of <= 16): one matrix tile */
} fd_path;

/*
 * Shape of one decode step.
 *   batch, num_q_heads, num_kv_heads, head_dim: B, Hq, Hkv, D; Hq % Hkv == 0.
 *   max_seq_len : upper bound on every L_b; the plan must cover it. Keys at
 *                 or past min(L_b, max_seq_len) are never part of a result.
 *   page_size   : 0 for a contiguous cache; for a paged one the keys per page,
 *                 a power of two from 16 to 256.
 *   num_pages   : paged only -- the pool size; a block-table entry outside
 *                 [0, num_pages) makes its keys count as masked.
 *   q_dtype, kv_dtype, out_dtype: fd_dtype; supported combinations are
 *                 f32/f32/f32, bf16/bf16/{bf16,f32} and bf16/fp8/{bf16,f32}.
 *   q_len       : query tokens per sequence, 1 .. 16 (0 is read as 1). q, out
 *                 and lse_out hold q_len * Hq rows per sequence, token-major:
 *                 row (b, t, h) is (b * q_len + t) * Hq + h.
 */
typedef struct fd_problem {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_seq_len;
  int32_t page_size;
  int32_t num_pages;
  int32_t q_dtype;
  int32_t kv_dtype;
  int32_t out_dtype;
  int32_t q_len;
} fd_problem;

/*
 * KV cache strides in elements; the head_dim axis is always contiguous.
 *   contiguous: key j of (b, kv head) is at  k + b*stride_outer + kvh*stride_head + j*stride_token
 *   paged     : page = block_table[b*block_table_stride + j/page_size],
 *               slot = j % page_size,
 *               key j is at k + page*stride_outer + kvh*stride_head + slot*stride_token
 * K and V share the layout.
 * k_scale, v_scale: device float [Hkv], the per-KV-head dequantisation scales
 * of an fp8 cache (required then; ignored for other dtypes).
 */
typedef struct fd_kv_layout {
  int64_t stride_outer;
  int64_t stride_head;
  int64_t stride_token;
  const float* k_scale;
  const float* v_scale;
} fd_kv_layout;

/* How the keys are cut into the pieces whose records the merge combines. */
typedef enum fd_mode {
  FD_MODE_SPLITS = 0,     /* fixed chunks: split s of every sequence is [s*chunk_len, (s+1)*chunk_len) */
  FD_MODE_BALANCED = 1    /* equal runs of key tiles per worker wave, whatever the sequence lengths */
} fd_mode;

/*
 * Plan of one decode step.
 *
 * FD_MODE_SPLITS: split s of sequence b covers keys [s*chunk_len,
 *   min((s+1)*chunk_len, L_b)); it is empty when s*chunk_len >= L_b.
 *   num_splits * chunk_len >= max_seq_len; chunk_len is a multiple of 16.
 *   Every output row gets exactly num_splits records.
 *
 * FD_MODE_BALANCED: a (sequence, KV head, row tile) triple is a segment of
 *   ceil(L_b / tile) key tiles; a row tile is a run of the KV head's
 *   q_len * group query rows (all of them on the MFMA path when they fit in
 *   16). The segments of all sequences are laid end to end and cut into
 *   `workers` equal runs of tiles, one per worker wave, so the work per wave
 *   does not depend on how ragged the lengths are. An output row gets one
 *   record per run that touches its segment.
 *   num_splits and chunk_len are unused; tile is the kernel's tile size and
 *   must be the value fd_plan_splits wrote.
 */
typedef struct fd_plan {
  int32_t num_splits;     /* FD_MODE_SPLITS: chunks per sequence */
  int32_t chunk_len;      /* FD_MODE_SPLITS: keys per chunk */
  int32_t path;           /* fd_path chosen for the partial kernel */
  int32_t mode;           /* fd_mode */
  int32_t workers;        /* FD_MODE_BALANCED: worker waves */
  int32_t tile;           /* FD_MODE_BALANCED: keys per tile */
  int32_t lead_workers;   /* FD_MODE_BALANCED: the first lead_workers workers ... */
  int32_t lead_pct;       /* ... take lead_pct % of another worker's share of
                             tiles (0: every worker the same share); 0 in
                             FD_MODE_SPLITS */
} fd_plan;

typedef void* fd_stream;

/*
 * fd_plan_splits -- choose the chunk count and the partial kernel.
 * [MERGE] "分块数量是一笔成本账": more chunks expose more independent work
 * but add partial records, launch work and merge cost, which can lose on
 * short contexts; its closing paragraph asks to pick the path by batch,
 * context, head_dim and device. [INFRA] 2.6 "Flash-Decoding 的 Split-K":
 * with a single query, a grid of batch x heads alone leaves compute units idle.
 *
 *   num_cus       : compute units to fill; <= 0 asks the current HIP device
 *                   (its CU count, and how many worker waves of the chosen
 *                   kernel fit on a CU at once).
 *   forced_splits : > 0 gives FD_MODE_SPLITS with that num_splits (chunk_len
 *                   = the smallest multiple of 16 that covers max_seq_len);
 *                   trailing splits may be empty. 0 gives FD_MODE_BALANCED
 *                   with W workers per CU: enough for 128 KiB of K/V loads in
 *                   flight per CU (two tiles per worker: W = ceil(128 KiB /
 *                   (2 * tile * head_dim * 2 * kv bytes))), at most the
 *                   kernel's resident waves per CU, and fewer workers in all
 *                   when the keys would give a worker under 256 of them.
 *                   A kernel that runs two worker waves per SIMD (8 per CU)
 *                   gets lead_workers = workers / 2 and lead_pct = 130: the
 *                   older wave of each SIMD wins most issue slots, so the
 *                   first-dispatched half takes the larger share.
 *   out           : written on success only; out->path is the kernel choice.
 * Pure host function when num_cus > 0 (8 resident waves per CU assumed).
 */
fd_status fd_plan_splits(const fd_problem* problem, int32_t num_cus, int32_t forced_splits, fd_plan* out);

/*
 * fd_workspace_size -- bytes of device workspace a (problem, plan) needs,
 * each section aligned to 256 bytes. Returns 0 for an invalid argument.
 * [MERGE] closing paragraphs: the workspace follows the chunk count.
 * Sections in order (J = segments per sequence: KV heads x row tiles, set by
 * the problem and the plan's path only; R = query rows per segment):
 *   counts   int32 [B * J]                  first, in every mode; written by
 *                                           fd_decode only (see there)
 *   FD_MODE_SPLITS (rows = B * q_len * Hq, in output-row order):
 *     O_part   float [rows][num_splits][D]   normalised chunk outputs
 *     LSE_part float [rows][num_splits]      chunk log-sum-exp (natural log,
 *                                            -inf for an empty chunk)
 *   FD_MODE_BALANCED (slots = B * J + workers - 1; the T tiles --
 *   ceil(L_b / tile) per segment -- laid end to end in (sequence, segment)
 *   order, go to the workers in runs: q1 each to the first lead_workers, q2
 *   each to the rest, q2 = ceil(100 T / (lead_workers * lead_pct +
 *   (workers - lead_workers) * 100)), q1 = ceil(q2 lead_pct / 100); with
 *   lead_pct 0, q1 = q2 = ceil(T / workers)):
 *     O_part   float [slots][R][D]           the piece of segment s that
 *     LSE_part float [slots][R]              worker w ran is slot s + w
 *     tiles    int32 [B + 1]                 running tile counts per sequence
 */
size_t fd_workspace_size(const fd_problem* problem, const fd_plan* plan);

/*
 * fd_decode_partial -- launch the per-chunk kernel ([INFRA] 2.6 online softmax
 * over the chunk's keys; [QA] 二 and 三 for the record it writes).
 *   q            : device, [B][q_len][Hq][D] contiguous, q_dtype.
 *   k, v         : device, laid out as *kv describes, kv_dtype.
 *   seq_lens     : device int32 [B], the key count L_b of each sequence
 *                  (the q_len new tokens included).
 *   seq_lens_host: host int32 [B] or NULL. When given, each q_len <= L_b <=
 *                  max_seq_len is checked (L_b < q_len, so that a query
 *                  token would see no key, -> FD_ERR_EMPTY_SEQUENCE).
 *   block_table  : device int32, row stride block_table_stride; NULL iff
 *                  page_size == 0. Entries past ceil(L_b/page_size) are never read.
 *   scale        : multiplies every q.k ([INFRA] 2.4: 1/sqrt(head_dim)).
 *   workspace    : device, >= fd_workspace_size(problem, plan) bytes, 256-byte
 *                  aligned; fully rewritten (every record, empty ones included).
 *   stream       : stream the kernel runs on.
 *   after_stream : NULL, or the stream of the previous user of the workspace
 *                  (e.g. the last combine); when it differs from stream, the
 *                  launch waits for the work queued on it so far.
 * Device side, a row that sees no key (n <= 0 in the formula at the top of
 * this file) has only empty records.
 */
fd_status fd_decode_partial(const fd_problem* problem, const fd_plan* plan, const void* q, const void* k,
                            const void* v, const fd_kv_layout* kv, const int32_t* seq_lens,
                            const int32_t* seq_lens_host, const int32_t* block_table,
                            int32_t block_table_stride, float scale, void* workspace, size_t workspace_bytes,
                            fd_stream stream, fd_stream after_stream);

/*
 * fd_decode_combine -- launch the merge kernel ([QA] 三; [MERGE]
 * "用 log-sum-exp 给块结果定权重"; [INFRA] 2.6 "Flash-Decoding 的 Split-K",
 * the reduction kernel). For each output row: M = max_s LSE_s,
 * w_s = exp(LSE_s - M) (0 for an empty chunk), out = sum_s w_s o_s / sum_s w_s.
 *   workspace     : as written by fd_decode_partial with the same problem/plan.
 *   out           : device, [B][q_len][Hq][D] contiguous, 16-byte aligned,
 *                   out_dtype (bf16 rounds to nearest even).
 *   lse_out       : device float [B][q_len][Hq] or NULL: the log-sum-exp of all
 *                   of the row's scores, M + log(sum_s w_s).
 *   partial_stream: NULL, or the stream fd_decode_partial ran on; when it
 *                   differs from stream, the merge waits for the work queued
 *                   on it so far ([MERGE] closing paragraphs: the merge must see
 *                   every chunk result before it reads any).
 * A row whose chunks are all empty (it sees no key) gets out = 0 and lse = -inf.
 */
fd_status fd_decode_combine(const fd_problem* problem, const fd_plan* plan, const void* workspace,
                            size_t workspace_bytes, void* out, float* lse_out, fd_stream stream,
                            fd_stream partial_stream);

/*
 * fd_decode -- one launch for the whole step: fd_decode_partial's arguments
 * plus fd_decode_combine's outputs. The partial kernel writes its records
 * with device-coherent stores, waits for them, and then counts them on their
 * segment's counter (the counts section of the workspace) with a device-scope
 * atomic; the wave or workgroup that completes a segment's count reads that
 * segment's records with device-coherent loads and merges them into out /
 * lse_out exactly as fd_decode_combine would, then sets the counter back to
 * zero. [MERGE]
 * closing paragraphs: the merge must see every chunk result before it reads
 * any -- here the counter is that dependency.
 *   Requirement: the counts section (the first 4 * B * J bytes, J as in
 *   fd_workspace_size) must be zero when fd_decode starts: allocate the
 *   workspace zeroed. Every fd_decode that completes leaves it zero again, and
 *   fd_decode_partial / fd_decode_combine never write it under any plan, so a
 *   workspace may alternate between the two-launch and the single-launch
 *   step. A later problem or path with a larger B * J reaches into what were
 *   records: zero the section again after such a change. Counts that are not
 *   zero make segments merge early or never, which gives wrong outputs (the
 *   kernels never read or write outside the workspace because of it).
 * Rows that see no key get out = 0 and lse = -inf. A segment that one wave
 * covers whole is written to out directly. Otherwise its merge runs at the
 * end of the wave (or workgroup) that completes it, after a device-coherent
 * write, a wait and an atomic round trip, so it adds to the tail of the
 * launch; on MI355X this single launch measured 0-24 % slower than
 * fd_decode_partial + fd_decode_combine on the shapes tried, least where
 * segments have few pieces.
 *   Limit: the in-kernel merge addresses a segment's records with 32-bit
 *   offsets (FD_ERR_UNSUPPORTED past them; use partial + combine).
 */
fd_status fd_decode(const fd_problem* problem, const fd_plan* plan, const void* q, const void* k, const void* v,
                    const fd_kv_layout* kv, const int32_t* seq_lens, const int32_t* seq_lens_host,
                    const int32_t* block_table, int32_t block_table_stride, float scale, void* workspace,
                    size_t workspace_bytes, void* out, float* lse_out, fd_stream stream, fd_stream after_stream);

/*
 * fd_decode_static -- for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It is fd_decode_partial followed by fd_decode_combine on
 * `stream`, with fd_decode_partial's arguments and fd_decode_combine's
 * outputs, but the records live in a workspace the library owns: a static
 * device array of FD_STATIC_WORKSPACE_BYTES on each GPU, held until the
 * process ends. The call allocates nothing. It uses the array of the GPU
 * that `stream` belongs to (the current GPU for the null stream), whose
 * device address is looked up on the first call for that GPU.
 *   Limit: fd_workspace_size(problem, plan) <= FD_STATIC_WORKSPACE_BYTES, else
 *   FD_ERR_WORKSPACE_TOO_SMALL before anything is launched (use the calls
 *   with a caller's workspace, or a plan with fewer records).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *   last call's records (nothing in it has to start at zero: each call
 *   rewrites every record it reads). Calls that overlap on one GPU -- on
 *   streams with no ordering between them -- race on the array and give
 *   wrong outputs; order them (one stream, or events).
 * Outputs and errors as fd_decode_partial and fd_decode_combine.
 */
#define FD_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
fd_status fd_decode_static(const fd_problem* problem, const fd_plan* plan, const void* q, const void* k,
                           const void* v, const fd_kv_layout* kv, const int32_t* seq_lens,
                           const int32_t* seq_lens_host, const int32_t* block_table, int32_t block_table_stride,
                           float scale, void* out, float* lse_out, fd_stream stream);

/* Static text for a status code. */
const char* fd_status_string(fd_status status);

/* Message for the last failed call on the calling thread ("" if none). */
const char* fd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
