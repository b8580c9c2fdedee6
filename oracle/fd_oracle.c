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
 * Multi-token decode (q_len > 1, the speculative-verification exception that
 * [INFRA] 2.5 makes to "decode needs no causal mask"): the q_len query tokens
 * of sequence b are its last q_len positions, L_b - q_len .. L_b - 1, whose
 * keys are already in the cache. Token t sits at position L_b - q_len + t and,
 * under the causal rule of [INFRA] 2.5 (a query sees a key iff the key's
 * position is not after its own), attends keys 0 <= j <= L_b - q_len + t. A
 * row is (b, i) with i = t * Hq + h; q_len = 1 is the plain decode step.
 *
 * Inputs are decoded exactly: fp32 -> double directly; bf16 -> (bits << 16)
 * reinterpreted as fp32 -> double; fp8 e4m3 (the "KV Quant" that the
 * [INFRA] 04 summary lists among KV-cache optimisations; OCP E4M3 encoding:
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, exponent field 0 is subnormal) -> its exact value. With
 * per-KV-head scales, a key element is decode(k) * k_scale[kv head] and a
 * value element decode(v) * v_scale[kv head], formed in fp64.
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
#define FDO_FP8_E4M3 2

#define FDO_OK 0
#define FDO_ERR_ARG (-1)
#define FDO_ERR_EMPTY (-4)
#define FDO_ERR_NOMEM (-6)

/* OCP E4M3: (-1)^s * 2^(e - 7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * (m/8) for
 * e == 0; e == 15 with m == 7 is NaN (the format has no infinities). */
static double fdo_e4m3(uint8_t byte) {
  int sign = byte >> 7;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

static double fdo_decode(const void* base, int64_t idx, int dtype) {
  if (dtype == FDO_F32) {
    return (double)((const float*)base)[idx];
  }
  if (dtype == FDO_FP8_E4M3) {
    return fdo_e4m3(((const uint8_t*)base)[idx]);
  }
  uint32_t word = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

/* Decode of every byte value, for the tests that pin the fp8 decoding. */
int fdo_decode_e4m3(const uint8_t* in, int64_t n, double* out) {
  if (!in || !out || n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fdo_e4m3(in[i]);
  return 0;
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
  int q_len;              /* query tokens per sequence, >= 1 */
  const float* k_scale;   /* [Hkv] or NULL (= 1) */
  const float* v_scale;
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

static double fdo_kscale(const fdo_args* a, int kvh) { return a->k_scale ? (double)a->k_scale[kvh] : 1.0; }
static double fdo_vscale(const fdo_args* a, int kvh) { return a->v_scale ? (double)a->v_scale[kvh] : 1.0; }

/* s_j = scale * <q[b,i,:], k_j>, as a sequential fp64 sum over d, where the
 * key element is its decoded value times the head's key scale. */
static double fdo_score(const fdo_args* a, int b, int i, int kvh, int64_t j) {
  int64_t qo = (int64_t)b * a->q_sb + (int64_t)i * a->q_sh;
  int64_t ko = fdo_row_offset(a, b, kvh, j);
  double ks = fdo_kscale(a, kvh);
  double dot = 0.0;
  for (int d = 0; d < a->D; ++d) {
    dot += fdo_decode(a->q, qo + d, a->q_dtype) * (fdo_decode(a->k, ko + d, a->kv_dtype) * ks);
  }
  return a->scale * dot;
}

/* Keys row (b, i) may see: [0, L_b - q_len + 1 + t) with t = i / Hq. */
static int64_t fdo_row_limit(const fdo_args* a, int b, int i) {
  return (int64_t)a->seq_lens[b] - a->q_len + 1 + i / a->Hq;
}

static int fdo_check(const fdo_args* a) {
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->D <= 0) return FDO_ERR_ARG;
  if (a->Hq % a->Hkv != 0) return FDO_ERR_ARG;
  if (!a->q || !a->k || !a->v || !a->seq_lens) return FDO_ERR_ARG;
  if (a->page_size > 0 && !a->block_table) return FDO_ERR_ARG;
  if (a->q_len < 1) return FDO_ERR_ARG;
  if ((a->q_dtype != FDO_F32 && a->q_dtype != FDO_BF16) ||
      (a->kv_dtype != FDO_F32 && a->kv_dtype != FDO_BF16 && a->kv_dtype != FDO_FP8_E4M3))
    return FDO_ERR_ARG;
  return FDO_OK;
}

/*
 * Softmax-weighted value average over keys [lo, hi) of one row, in the plain
 * two-pass form: scores, then max, then exp-sum and weighted sum.
 * Writes out[D] and returns log-sum-exp. Requires hi > lo.
 */
static double fdo_softmax_average(const fdo_args* a, int b, int i, int kvh, int64_t lo, int64_t hi,
                                  double* scores, double* out) {
  for (int64_t j = lo; j < hi; ++j) scores[j - lo] = fdo_score(a, b, i, kvh, j);
  double m = scores[0];
  for (int64_t j = lo + 1; j < hi; ++j)
    if (scores[j - lo] > m) m = scores[j - lo];
  double z = 0.0;
  for (int d = 0; d < a->D; ++d) out[d] = 0.0;
  for (int64_t j = lo; j < hi; ++j) {
    double w = exp(scores[j - lo] - m);
    z += w;
    int64_t vo = fdo_row_offset(a, b, kvh, j);
    for (int d = 0; d < a->D; ++d) out[d] += w * (fdo_decode(a->v, vo + d, a->kv_dtype) * fdo_vscale(a, kvh));
  }
  for (int d = 0; d < a->D; ++d) out[d] /= z;
  return m + log(z);
}

/* Row r as (b, i): the given pair, or the r-th of all B * q_len * Hq rows. */
static void fdo_row_ids(const int32_t* rows, int64_t r, int64_t per_seq, int* b, int* i) {
  if (rows) {
    *b = rows[2 * r];
    *i = rows[2 * r + 1];
  } else {
    *b = (int)(r / per_seq);
    *i = (int)(r % per_seq);
  }
}

/*
 * Plain definition. q row i of sequence b is at q + b*q_sb + i*q_sh
 * (i = t*Hq + h). rows: NULL for all B*q_len*Hq rows in (b, t, h) order,
 * else nrows pairs (b, i). k_scale / v_scale: [Hkv] or NULL.
 * out: [nrows][D], lse: [nrows] (may be NULL).
 * Returns FDO_ERR_EMPTY if a requested row sees no key (the merge of
 * [MERGE]'s example refuses "no valid blocks"), FDO_ERR_ARG on bad arguments.
 */
int fdo_attention_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb, int64_t q_sh,
                      const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh, int64_t st,
                      const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride, int page_size,
                      double scale, int q_len, const float* k_scale, const float* v_scale, const int32_t* rows,
                      int64_t nrows, double* out, double* lse) {
  fdo_args a = {B, Hq, Hkv, D, q, q_dtype, q_sb, q_sh, k, v, kv_dtype, so, sh, st,
                seq_lens, block_table, bt_stride, page_size, scale, q_len, k_scale, v_scale};
  int rc = fdo_check(&a);
  if (rc != FDO_OK) return rc;
  if (!out) return FDO_ERR_ARG;
  const int64_t per_seq = (int64_t)q_len * Hq;
  if (!rows) nrows = (int64_t)B * per_seq;
  for (int64_t r = 0; r < nrows; ++r) {
    int b, i;
    fdo_row_ids(rows, r, per_seq, &b, &i);
    if (b < 0 || b >= B || i < 0 || i >= per_seq) return FDO_ERR_ARG;
    if (fdo_row_limit(&a, b, i) <= 0) return FDO_ERR_EMPTY;
  }
  int status = FDO_OK;
  int g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int b, i;
    fdo_row_ids(rows, r, per_seq, &b, &i);
    int64_t L = fdo_row_limit(&a, b, i);
    double* scores = (double*)malloc(sizeof(double) * (size_t)L);
    if (!scores) {
#pragma omp atomic write
      status = FDO_ERR_NOMEM;
      continue;
    }
    double l = fdo_softmax_average(&a, b, i, (i % Hq) / g, 0, L, scores, out + r * D);
    if (lse) lse[r] = l;
    free(scores);
  }
  return status;
}

/*
 * Chunk-and-merge form for one partition of the key range, applied to every
 * row: chunk c covers keys [cuts[c], cuts[c+1]) intersected with the keys the
 * row sees, [0, L_b - q_len + 1 + t).
 * cuts has nchunks+1 ascending entries with cuts[0] == 0. Outputs:
 *   part_o [nrows][nchunks][D], part_lse [nrows][nchunks]  (may be NULL)
 *   out [nrows][D], lse [nrows] (lse may be NULL)
 * Empty chunks give part_o = 0, part_lse = -inf and weight 0.
 */
int fdo_attention_chunked_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb,
                              int64_t q_sh, const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh,
                              int64_t st, const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride,
                              int page_size, double scale, int q_len, const float* k_scale,
                              const float* v_scale, const int32_t* rows, int64_t nrows, const int64_t* cuts,
                              int nchunks, double* part_o, double* part_lse, double* out, double* lse) {
  fdo_args a = {B, Hq, Hkv, D, q, q_dtype, q_sb, q_sh, k, v, kv_dtype, so, sh, st,
                seq_lens, block_table, bt_stride, page_size, scale, q_len, k_scale, v_scale};
  int rc = fdo_check(&a);
  if (rc != FDO_OK) return rc;
  if (!out || !cuts || nchunks <= 0 || cuts[0] != 0) return FDO_ERR_ARG;
  for (int i = 0; i < nchunks; ++i)
    if (cuts[i + 1] < cuts[i]) return FDO_ERR_ARG;
  const int64_t per_seq = (int64_t)q_len * Hq;
  if (!rows) nrows = (int64_t)B * per_seq;
  for (int64_t r = 0; r < nrows; ++r) {
    int b, i;
    fdo_row_ids(rows, r, per_seq, &b, &i);
    if (b < 0 || b >= B || i < 0 || i >= per_seq) return FDO_ERR_ARG;
    if (fdo_row_limit(&a, b, i) <= 0) return FDO_ERR_EMPTY;
    if (cuts[nchunks] < seq_lens[b]) return FDO_ERR_ARG;
  }
  int status = FDO_OK;
  int g = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    int b, qi;
    fdo_row_ids(rows, r, per_seq, &b, &qi);
    int64_t L = fdo_row_limit(&a, b, qi);
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
        pl[i] = fdo_softmax_average(&a, b, qi, (qi % Hq) / g, lo, hi, scores, po + (int64_t)i * D);
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

/* Sets that thread count (for timing the oracle on one core). */
void fdo_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
