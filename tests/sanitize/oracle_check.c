/*
 * oracle_check.c -- drives the fp64 oracle (oracle/fd_oracle.c) on small
 * inputs in a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * TEST INFRASTRUCTURE ONLY (run by tests/test_host_sanitizers.py on the CPU).
 *
 * Buffers are allocated at exactly the size the inputs need, so that a read
 * past a sequence's keys, a block table row or a scale array is a heap
 * overflow the sanitizer reports. Checks, besides a clean run:
 *   - the worked example of www.2kiu.com/news/6053916 ("用 log-sum-exp 给块结果
 *     定权重"): scores [0, 0, 10], values [0, 0, 9] give 9 / (1 + 2 e^-10),
 *     split 2 | 1 or not;
 *   - the chunked form equals the plain one (1e-12 relative) on random
 *     contiguous and paged, fp32 / bf16 / fp8, one- and three-token inputs
 *     with NaN stored past every sequence's keys;
 *   - a row that sees no key and malformed arguments are refused.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int fdo_attention_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb, int64_t q_sh,
                      const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh, int64_t st,
                      const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride, int page_size,
                      double scale, int q_len, const float* k_scale, const float* v_scale, const int32_t* rows,
                      int64_t nrows, double* out, double* lse);
int fdo_attention_chunked_f64(int B, int Hq, int Hkv, int D, const void* q, int q_dtype, int64_t q_sb,
                              int64_t q_sh, const void* k, const void* v, int kv_dtype, int64_t so, int64_t sh,
                              int64_t st, const int32_t* seq_lens, const int32_t* block_table, int64_t bt_stride,
                              int page_size, double scale, int q_len, const float* k_scale, const float* v_scale,
                              const int32_t* rows, int64_t nrows, const int64_t* cuts, int nchunks,
                              double* part_o, double* part_lse, double* out, double* lse);

static int failures = 0;
#define CHECK(cond, ...)                                \
  do {                                                  \
    if (!(cond)) {                                      \
      if (failures < 20) {                              \
        fprintf(stderr, "FAIL: " __VA_ARGS__);          \
        fprintf(stderr, "\n");                          \
      }                                                 \
      ++failures;                                       \
    }                                                   \
  } while (0)

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32(void) {   /* xorshift64 */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 32);
}
static float uniform(void) { return (float)((next_u32() >> 8) * (1.0 / 16777216.0)) * 2.0f - 1.0f; }

/* Element e of a buffer of dtype dt (0 fp32, 1 bf16, 2 fp8) set from x; NaN when nan. */
static void put(void* buf, int64_t e, int dt, float x, int nan) {
  if (dt == 0) {
    ((float*)buf)[e] = nan ? NAN : x;
  } else if (dt == 1) {
    uint32_t w;
    float f = nan ? NAN : x;
    memcpy(&w, &f, 4);
    ((uint16_t*)buf)[e] = (uint16_t)(w >> 16);
  } else {
    uint8_t code = nan ? 0x7f : (uint8_t)(next_u32() & 0xff);
    if (!nan && (code & 0x7f) == 0x7f) code &= 0xfe;   /* keep valid keys finite */
    ((uint8_t*)buf)[e] = code;
  }
}

static size_t esize(int dt) { return dt == 0 ? 4 : dt == 1 ? 2 : 1; }

static void counterexample(void) {
  float q = 1.0f, k[3] = {0.0f, 0.0f, 10.0f}, v[3] = {0.0f, 0.0f, 9.0f};
  int32_t len = 3;
  double out, lse, po[2], pl[2], out_c, lse_c;
  int64_t cuts[3] = {0, 2, 3};
  int rc = fdo_attention_f64(1, 1, 1, 1, &q, 0, 1, 1, k, v, 0, 3, 3, 1, &len, NULL, 0, 0, 1.0, 1, NULL, NULL,
                             NULL, 1, &out, &lse);
  CHECK(rc == 0, "counterexample rc %d", rc);
  const double closed = 9.0 / (1.0 + 2.0 * exp(-10.0));
  CHECK(fabs(out - closed) <= 1e-14 * closed, "counterexample out %.17g", out);
  rc = fdo_attention_chunked_f64(1, 1, 1, 1, &q, 0, 1, 1, k, v, 0, 3, 3, 1, &len, NULL, 0, 0, 1.0, 1, NULL, NULL,
                                 NULL, 1, cuts, 2, po, pl, &out_c, &lse_c);
  CHECK(rc == 0 && po[0] == 0.0 && po[1] == 9.0 && pl[1] == 10.0, "counterexample chunks");
  CHECK(fabs(pl[0] - log(2.0)) <= 1e-15, "counterexample chunk 0 lse");
  CHECK(fabs(out_c - out) <= 1e-12 * out && fabs(lse_c - lse) <= 1e-12 * lse, "counterexample merge");
}

/* One random problem: chunked == plain on every row. */
static void random_case(int B, int Hq, int Hkv, int D, int dt, int q_len, int page) {
  int32_t* lens = malloc(sizeof(int32_t) * B);
  int maxl = 0, total_pages = 0, max_pages = 0;
  for (int b = 0; b < B; ++b) {
    lens[b] = b == 0 ? 50 + q_len : q_len + (int)(next_u32() % 70);   /* the longest is past every cut */
    if (lens[b] > maxl) maxl = lens[b];
    if (page) {
      int n = (lens[b] + page - 1) / page;
      total_pages += n;
      if (n > max_pages) max_pages = n;
    }
  }
  const int qdt = dt == 2 ? 1 : dt;
  const int64_t rows = (int64_t)B * q_len * Hq;
  void* q = malloc(esize(qdt) * rows * D);
  for (int64_t e = 0; e < rows * D; ++e) put(q, e, qdt, uniform(), 0);
  int64_t so, sh = 0, st = D, slots;
  int32_t* table = NULL;
  if (page) {
    sh = (int64_t)page * D;
    so = (int64_t)Hkv * sh;
    slots = (int64_t)total_pages * Hkv * page;
    table = malloc(sizeof(int32_t) * B * max_pages);
    int* perm = malloc(sizeof(int) * total_pages);
    for (int i = 0; i < total_pages; ++i) perm[i] = i;
    for (int i = total_pages - 1; i > 0; --i) {
      int j = (int)(next_u32() % (uint32_t)(i + 1)), t = perm[i];
      perm[i] = perm[j];
      perm[j] = t;
    }
    int pos = 0;
    for (int b = 0; b < B; ++b)
      for (int p = 0; p < max_pages; ++p)
        table[b * max_pages + p] = p < (lens[b] + page - 1) / page ? perm[pos++] : -1;
    free(perm);
  } else {
    sh = (int64_t)maxl * D;
    so = (int64_t)Hkv * sh;
    slots = (int64_t)B * Hkv * maxl;
  }
  void* k = malloc(esize(dt) * slots * D);
  void* v = malloc(esize(dt) * slots * D);
  for (int64_t e = 0; e < slots * D; ++e) {
    put(k, e, dt, 0.0f, 1);   /* NaN everywhere first: padding stays NaN */
    put(v, e, dt, 0.0f, 1);
  }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hkv; ++h)
      for (int j = 0; j < lens[b]; ++j) {
        int64_t row = page ? (int64_t)table[b * max_pages + j / page] * so + h * sh + (j % page) * st
                           : (int64_t)b * so + h * sh + (int64_t)j * st;
        for (int d = 0; d < D; ++d) {
          put(k, row + d, dt, 2.0f * uniform(), 0);
          put(v, row + d, dt, uniform(), 0);
        }
      }
  float* ks = malloc(sizeof(float) * Hkv);
  float* vs = malloc(sizeof(float) * Hkv);
  for (int h = 0; h < Hkv; ++h) {
    ks[h] = 0.01f + 0.02f * (float)h;
    vs[h] = 0.03f + 0.01f * (float)h;
  }
  const float* kscale = dt == 2 ? ks : NULL;
  const float* vscale = dt == 2 ? vs : NULL;
  double* out = malloc(sizeof(double) * rows * D);
  double* lse = malloc(sizeof(double) * rows);
  const int nch = 5;
  int64_t cuts[6] = {0, 1, 17, 18, 40, 0};
  cuts[5] = maxl;
  double* po = malloc(sizeof(double) * rows * nch * D);
  double* pl = malloc(sizeof(double) * rows * nch);
  double* out_c = malloc(sizeof(double) * rows * D);
  double* lse_c = malloc(sizeof(double) * rows);
  const double scale = 1.0 / sqrt((double)D);
  int rc = fdo_attention_f64(B, Hq, Hkv, D, q, qdt, (int64_t)q_len * Hq * D, D, k, v, dt, so, sh, st, lens, table,
                             max_pages, page, scale, q_len, kscale, vscale, NULL, rows, out, lse);
  CHECK(rc == 0, "plain rc %d (B %d dt %d page %d)", rc, B, dt, page);
  rc = fdo_attention_chunked_f64(B, Hq, Hkv, D, q, qdt, (int64_t)q_len * Hq * D, D, k, v, dt, so, sh, st, lens,
                                 table, max_pages, page, scale, q_len, kscale, vscale, NULL, rows, cuts, nch, po, pl,
                                 out_c, lse_c);
  CHECK(rc == 0, "chunked rc %d", rc);
  for (int64_t r = 0; r < rows; ++r) {
    double mx = 0.0, err = 0.0;
    for (int d = 0; d < D; ++d) {
      CHECK(isfinite(out[r * D + d]), "non-finite output row %ld", (long)r);
      if (fabs(out[r * D + d]) > mx) mx = fabs(out[r * D + d]);
      if (fabs(out[r * D + d] - out_c[r * D + d]) > err) err = fabs(out[r * D + d] - out_c[r * D + d]);
    }
    CHECK(err <= 1e-12 * mx, "row %ld chunked vs plain %.3g", (long)r, err / mx);
    CHECK(fabs(lse[r] - lse_c[r]) <= 1e-12 * fmax(1.0, fabs(lse[r])), "row %ld lse", (long)r);
  }
  /* A row that sees no key is refused. */
  int32_t keep = lens[0];
  lens[0] = q_len - 1;
  rc = fdo_attention_f64(B, Hq, Hkv, D, q, qdt, (int64_t)q_len * Hq * D, D, k, v, dt, so, sh, st, lens, table,
                         max_pages, page, scale, q_len, kscale, vscale, NULL, rows, out, lse);
  CHECK(rc == -4, "empty row rc %d", rc);
  lens[0] = keep;
  rc = fdo_attention_f64(B, Hq + 1, Hkv, D, q, qdt, 0, 0, k, v, dt, so, sh, st, lens, table, max_pages, page, scale,
                         q_len, kscale, vscale, NULL, rows, out, lse);
  CHECK(rc == -1 || Hq + 1 == Hkv, "bad group rc %d", rc);
  free(lens); free(q); free(k); free(v); free(table); free(ks); free(vs);
  free(out); free(lse); free(po); free(pl); free(out_c); free(lse_c);
}

int main(void) {
  counterexample();
  const int dts[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int page = 0; page <= 32; page += 16)
      for (int q_len = 1; q_len <= 3; q_len += 2) {
        random_case(3, 4, 2, 16, dts[i], q_len, page);
        random_case(2, 3, 3, 8, dts[i], q_len, page);
      }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle_check: ok\n");
  return 0;
}
