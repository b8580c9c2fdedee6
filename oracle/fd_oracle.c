/*
 * fd_oracle.c -- plain fp64 CPU oracle for single-query (decode-step) attention.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library. The GPU library never includes,
 * links or calls anything here, and this file includes nothing of it.
 *
 * Pages cited (by title and section):
 *   [QA]    "FlashDecoding面经-vivj啥关系 vi就是原来的O呗用LSE是为了防止溢出吗"
 *           (www.gtnt.cn/news/53829), parts 一 / 二 / 三.
 *   [MERGE] the www.2kiu.com/news/6053916 article, sections
 *           "用 log-sum-exp 给块结果定权重" (with its Python example) and
 *           "为什么这个反例特别容易看出平均法错误".
 *   [INFRA] "AI Infra：深入理解大模型中的数学与Infra优化", sections 2.3
 *           (safe softmax), 2.4 (scaling by 1/sqrt(d_k)), 2.5 (masking),
 *           2.6 (online softmax, "LSE 与 Online Softmax",
 *           "Flash-Decoding 的 Split-K").
 *
 * Two entry points:
 *
 *   fdo_attention_f64   -- the plain definition. For every requested row
 *     (batch b, query head h):
 *         g      = Hq / Hkv,   kv head = h / g    (contiguous query groups)
 *         s_j    = scale * sum_d q[b,h,d] * k[b, kv head, j, d],  0 <= j < L_b
 *         m      = max_j s_j
 *         w_j    = exp(s_j - m),   Z = sum_j w_j
 *         out[d] = (sum_j w_j * v[b, kv head, j, d]) / Z
 *         lse    = m + log(Z)
 *     The scale is [INFRA] 2.4; subtracting the max is [INFRA] 2.3; keys at or
 *     past L_b are simply not part of the sums ([INFRA] 2.5: masked keys leave
 *     numerator and denominator); lse is the log-sum-exp of [INFRA] 2.6
 *     "LSE 与 Online Softmax". Every sum is a sequential fp64 sum in index
 *     order; nothing is blocked, fused or reordered.
 *
 *   fdo_attention_chunked_f64 -- the chunk-and-merge algorithm of [MERGE]
 *     "用 log-sum-exp 给块结果定权重" and [QA] parts 二 and 三, for one given
 *     partition of the key range. Each non-empty chunk i gets its own
 *         m_i, l_i = sum exp(s_j - m_i),
 *         o_i = (sum exp(s_j - m_i) v_j) / l_i     (the normalised output)
 *         LSE_i = m_i + log(l_i)
 *     and the merge is
 *         M = max_i LSE_i,  w_i = exp(LSE_i - M),
 *         out = sum_i w_i o_i / sum_i w_i,   lse = M + log(sum_i w_i).
 *     An empty chunk (no valid key) gets o_i = 0, LSE_i = -inf and weight 0:
 *     [MERGE] forbids turning it into a "zero output, normal weight" block.
 *     It exists to pin the merge algebra against the plain definition.
 *
 * Inputs are decoded exactly: fp32 -> double directly; bf16 -> (bits << 16)
 * reinterpreted as fp32 -> double.
 *
 * KV addressing, in elements, D innermost and contiguous:
 *   contiguous (page_size == 0): k + b*so + kvh*sh + j*st
 *   paged      (page_size  > 0): page = block_table[b*bt_stride + j/page_size],
 *                                k + page*so + kvh*sh + (j % page_size)*st
 * Logical order is kept: key j is always the j-th key of the sequence,
 * whatever page holds it ([MERGE] "分块数量是一笔成本账", paragraph on masks
 * and paging; [INFRA] 2.5, block-table gather).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FDO_F32 0
#define FDO_BF16 1

#define FDO_OK 0
#define FDO_ERR_ARG (-1)
#define FDO_ERR_EMPTY (-4)
#define FDO_ERR_NOMEM (-6)

static double fdo_decode(const void* base, int64_t idx, int dtype) {
  if (dtype == FDO_F32) {
    return (double)((const float*)base)[idx];
  }
  uint32_t word = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

typedef struct {
  int B, Hq, Hkv, D;
  const void* q;
  int q_dtype;
  int64_t q_sb, q_sh;
  const void* k;
  const void* v;
  int kv_dtype;
  int64_t so, sh, st;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int64_t bt_stride;
  int page_size;
  double scale;
} fdo_args;

/* Element offset of key/value row j of (b, kv head). */
static int64_t fdo_row_offset(const fdo_args* a, int b, int kvh, int64_t j) {
  if (a->page_size > 0) {
    int64_t page = a->block_table[(int64_t)b * a->bt_stride + j / a->page_size];
    int64_t slot = j % a->page_size;
    return page * a->so + (int64_t)kvh * a->sh + slot * a->st;
  }
  return (int64_t)b * a->so + (int64_t)kvh * a->sh + j * a->st;
}

/* s_j = scale * <q[b,h,:], k_j>, as a sequential fp64 sum over d. */
static double fdo_score(const fdo_args* a, int b, int h, int kvh, int64_t j) {
  int64_t qo = (int64_t)b * a->q_sb + (int64_t)h * a->q_sh;
  int64_t ko = fdo_row_offset(a, b, kvh, j);
  double dot = 0.0;
  for (int d = 0; d < a->D; ++d) {
    dot += fdo_decode(a->q, qo + d, a->q_dtype) * fdo_decode(a->k, ko + d, a->kv_dtype);
  }
  return a->scale * dot;
}

static int fdo_check(const fdo_args* a) {
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->D <= 0) return FDO_ERR_ARG;
  if (a->Hq % a->Hkv != 0) return FDO_ERR_ARG;
  if (!a->q || !a->k || !a->v || !a->seq_lens) return FDO_ERR_ARG;
  if (a->page_size > 0 && !a->block_table) return FDO_ERR_ARG;
  if ((a->q_dtype != FDO_F32 && a->q_dtype != FDO_BF16) ||
      (a->kv_dtype != FDO_F32 && a->kv_dtype != FDO_BF16))
    return FDO_ERR_ARG;
  return FDO_OK;
}

/*
 * Softmax-weighted value average over keys [lo, hi) of one row, in the plain
 * two-pass form: scores, then max, then exp-sum and weighted sum.
 * Writes out[D] and returns log-sum-exp. Requires hi > lo.
 */
static double fdo_softmax_average(const fdo_args* a, int b, int h, int kvh, int64_t lo, int64_t hi,
                                  double* scores, double* out) {
  for (int64_t j = lo; j < hi; ++j) scores[j - lo] = fdo_score(a, b, h, kvh, j);
  double m = scores[0];
  for (int64_t j = lo + 1; j < hi; ++j)
    if (scores[j - lo] > m) m = scores[j - lo];
  double z = 0.0;
  for (int d = 0; d < a->D; ++d) out[d] = 0.0;
  for (int64_t j = lo; j < hi; ++j) {
    double w = exp(scores[j - lo] - m);
    z += w;
    int64_t vo = fdo_row_offset(a, b, kvh, j);
    for (int d = 0; d < a->D; ++d) out[d] += w * fdo_decode(a->v, vo + d, a->kv_dtype);
  }
  for (int d = 0; d < a->D; ++d) out[d] /= z;
  return m + log(z);
}

static void fdo_row_ids(const int32_t* rows, int64_t r, int Hq, int* b, int* h) {
  if (rows) {
    *b = rows[2 * r];
    *h = rows[2 * r + 1];
  } else {
    *b = (int)(r / Hq);
    *h = (int)(r % Hq);
  }
}

/*
 * Plain definition. rows: NULL for all B*Hq rows in (b, h) order, else
 * nrows pairs (b, h). out: [nrows][D], lse: [nrows] (may be NULL).
 * Returns FDO_ERR_EMPTY if a requested row has L_b <= 0 (the merge of
 * [MERGE]'s example refuses "no valid blocks"), FDO_ERR_ARG on bad arguments.
 */
int fdo_attention_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb, int64_t q_sh,
                      const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh, int64_t st,
                      const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride, int page_size,
                      double scale, const int32_t* rows, int64_t nrows, double* out, double* lse) {
  fdo_args a = {B, Hq, Hkv, D, q, q_dtype, q_sb, q_sh, k, v, kv_dtype, so, sh, st,
                seq_lens, block_table, bt_stride, page_size, scale};
  int rc = fdo_check(&a);
  if (rc != FDO_OK) return rc;
  if (!out) return FDO_ERR_ARG;
  if (!rows) nrows = (int64_t)B * Hq;
  for (int64_t r = 0; r < nrows; ++r) {
    int b, h;
    fdo_row_ids(rows, r, Hq, &b, &h);
    if (b < 0 || b >= B || h < 0 || h >= Hq) return FDO_ERR_ARG;
    if (seq_lens[b] <= 0) return FDO_ERR_EMPTY;
  }
  int status = FDO_OK;
  int g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int b, h;
    fdo_row_ids(rows, r, Hq, &b, &h);
    int64_t L = seq_lens[b];
    double* scores = (double*)malloc(sizeof(double) * (size_t)L);
    if (!scores) {
#pragma omp atomic write
      status = FDO_ERR_NOMEM;
      continue;
    }
    double l = fdo_softmax_average(&a, b, h, h / g, 0, L, scores, out + r * D);
    if (lse) lse[r] = l;
    free(scores);
  }
  return status;
}

/*
 * Chunk-and-merge form for one partition of the key range, applied to every
 * row: chunk i covers keys [cuts[i], cuts[i+1]) intersected with [0, L_b).
 * cuts has nchunks+1 ascending entries with cuts[0] == 0. Outputs:
 *   part_o [nrows][nchunks][D], part_lse [nrows][nchunks]  (may be NULL)
 *   out [nrows][D], lse [nrows] (lse may be NULL)
 * Empty chunks give part_o = 0, part_lse = -inf and weight 0.
 */
int fdo_attention_chunked_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb,
                              int64_t q_sh, const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh,
                              int64_t st, const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride,
                              int page_size, double scale, const int32_t* rows, int64_t nrows,
                              const int64_t* cuts, int nchunks, double* part_o, double* part_lse, double* out,
                              double* lse) {
  fdo_args a = {B, Hq, Hkv, D, q, q_dtype, q_sb, q_sh, k, v, kv_dtype, so, sh, st,
                seq_lens, block_table, bt_stride, page_size, scale};
  int rc = fdo_check(&a);
  if (rc != FDO_OK) return rc;
  if (!out || !cuts || nchunks <= 0 || cuts[0] != 0) return FDO_ERR_ARG;
  for (int i = 0; i < nchunks; ++i)
    if (cuts[i + 1] < cuts[i]) return FDO_ERR_ARG;
  if (!rows) nrows = (int64_t)B * Hq;
  for (int64_t r = 0; r < nrows; ++r) {
    int b, h;
    fdo_row_ids(rows, r, Hq, &b, &h);
    if (b < 0 || b >= B || h < 0 || h >= Hq) return FDO_ERR_ARG;
    if (seq_lens[b] <= 0) return FDO_ERR_EMPTY;
    if (cuts[nchunks] < seq_lens[b]) return FDO_ERR_ARG;
  }
  int status = FDO_OK;
  int g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int b, h;
    fdo_row_ids(rows, r, Hq, &b, &h);
    int64_t L = seq_lens[b];
    double* scores = (double*)malloc(sizeof(double) * (size_t)L);
    double* po = (double*)malloc(sizeof(double) * (size_t)nchunks * (size_t)D);
    double* pl = (double*)malloc(sizeof(double) * (size_t)nchunks);
    if (!scores || !po || !pl) {
#pragma omp atomic write
      status = FDO_ERR_NOMEM;
      free(scores);
      free(po);
      free(pl);
      continue;
    }
    /* Per-chunk partials: the normalised output and its log-sum-exp. */
    for (int i = 0; i < nchunks; ++i) {
      int64_t lo = cuts[i] < L ? cuts[i] : L;
      int64_t hi = cuts[i + 1] < L ? cuts[i + 1] : L;
      if (hi > lo) {
        pl[i] = fdo_softmax_average(&a, b, h, h / g, lo, hi, scores, po + (int64_t)i * D);
      } else {
        for (int d = 0; d < D; ++d) po[(int64_t)i * D + d] = 0.0;
        pl[i] = -INFINITY;
      }
    }
    /* Merge: weights exp(LSE_i - max LSE), empty chunks weigh zero. */
    double M = -INFINITY;
    for (int i = 0; i < nchunks; ++i)
      if (pl[i] > M) M = pl[i];
    double wsum = 0.0;
    double* o = out + r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int i = 0; i < nchunks; ++i) {
      if (pl[i] == -INFINITY) continue;
      double w = exp(pl[i] - M);
      wsum += w;
      for (int d = 0; d < D; ++d) o[d] += w * po[(int64_t)i * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= wsum;
    if (lse) lse[r] = M + log(wsum);
    if (part_o) memcpy(part_o + r * (int64_t)nchunks * D, po, sizeof(double) * (size_t)nchunks * (size_t)D);
    if (part_lse) memcpy(part_lse + r * (int64_t)nchunks, pl, sizeof(double) * (size_t)nchunks);
    free(scores);
    free(po);
    free(pl);
  }
  return status;
}

/* Threads the OpenMP runtime will use for the loops above. */
int fdo_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
