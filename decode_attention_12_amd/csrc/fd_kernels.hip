// fd_kernels.hip -- gfx950 kernels for split-KV decode attention.
//
// Pages cited (by title and section):
//   [QA]    "FlashDecoding面经-vivj啥关系 vi就是原来的O呗用LSE是为了防止溢出吗",
//           parts 二 (a chunk writes acc_i / l_i, its locally normalised
//           output) and 三 (LSE_i = m_i + log l_i; weights exp(LSE_i - max)).
//   [MERGE] www.2kiu.com/news/6053916, "用 log-sum-exp 给块结果定权重" (an empty
//           chunk must not become a zero output with normal weight) and
//           "分块数量是一笔成本账" (masks consistent across chunks; paged
//           logical order).
//   [INFRA] "AI Infra：深入理解大模型中的数学与Infra优化", 2.3 (subtract the
//           max), 2.4 (scale), 2.5 (masked keys leave numerator and
//           denominator; block-table gather), 2.6 (online softmax: running
//           max, rescale by exp(m_old - m_new), the (m, l, O) state; "LSE 与
//           Online Softmax": P = exp2 after one FMA; "Flash-Decoding 的
//           Split-K": each chunk writes its local O and LSE, a reduction
//           kernel merges them).
//
// Work split. One workgroup of four waves owns one (split, KV head, sequence)
// and every query head that reads that KV head, so each K/V byte of the chunk
// is fetched from HBM once. The waves take 32-key (or 16/64-key) tiles of the
// chunk in turn, each keeping its own online-softmax state in registers; the
// four states are merged through LDS with the same LSE algebra at the end.
//
// Scores are kept in base-2 units: q.k is multiplied by scale*log2(e), so the
// exponentials are single v_exp_f32 (2^x) instructions; the chunk LSE is
// converted back to the natural log when it is written.
//
// Masking: a key at or past hi = min(L_b, end of chunk), or on a page whose
// block-table entry is outside the pool, gets score -inf and so weight 0.
// K/V come in through buffer loads whose range ends at key hi, so such keys
// read as zeros (never NaN into p*v), no load leaves the valid part of the
// cache, and block-table entries past the sequence's last page are never read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Element access goes through these by-value helpers: hipcc 7.2 folds
// __builtin_bit_cast applied directly to an ext_vector element (v[i]) into
// element 0 of the vector.
__device__ __forceinline__ float as_f32(uint32_t w) { return __builtin_bit_cast(float, w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DPP lane moves inside a 16-lane row.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;       // row_ror:4
constexpr int kRowRor8 = 0x128;       // row_ror:8
constexpr int kRowHalfMirror = 0x141; // reverse each half row of 8 lanes

// Sum over aligned groups of kLanes lanes; every lane of the group gets it.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(kLanes == 8 || kLanes == 16 || kLanes == 32, "group size");
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if constexpr (kLanes == 8) {
    x += dpp<kRowHalfMirror>(x);
  } else {
    x += dpp<kRowRor4>(x);
    x += dpp<kRowRor8>(x);
    if constexpr (kLanes == 32) x += __shfl_xor(x, 16);
  }
  return x;
}

// Reduce across the groups: lanes l, l ^ kStride, l ^ 2kStride, ... (< 64).
template <int kStride>
__device__ __forceinline__ float across_sum(float x) {
#pragma unroll
  for (int s = kStride; s < 64; s <<= 1) x += __shfl_xor(x, s);
  return x;
}
template <int kStride>
__device__ __forceinline__ float across_max(float x) {
#pragma unroll
  for (int s = kStride; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}

__device__ __forceinline__ int clamp_len(const PartialLaunch& a, int b) {
  int L = a.seq_lens[b];
  return min(max(L, 0), a.max_seq_len);
}

// Buffer descriptors for the K and V rows of (sequence b, KV head kvh).
// Contiguous: one pair for the chunk, based at key lo. Paged: one pair per
// 16-key page. num_records covers only keys below hi, so a row at or past hi
// (and every row of an out-of-pool page) reads as zeros: masked keys carry
// finite values into the arithmetic, and no load leaves the valid part of the
// cache. Loads go through a fixed 32-bit lane offset plus an SGPR offset.
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family descriptor word 3
constexpr int kStreamLoad = 2;             // nontemporal: every K/V byte is read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, kBufferWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, kStreamLoad));
}

template <bool kPaged>
struct KvSource {
  const PartialLaunch& a;
  int b, kvh, lo, hi, esz, row_bytes;
  __amdgpu_buffer_rsrc_t kc, vc;   // contiguous: the chunk's descriptors

  __device__ KvSource(const PartialLaunch& a_, int b_, int kvh_, int lo_, int hi_, int esz_)
      : a(a_), b(b_), kvh(kvh_), lo(lo_), hi(hi_), esz(esz_), row_bytes((int)a_.stride_token * esz_) {
    if constexpr (!kPaged) {
      const int64_t base = ((int64_t)b * a.stride_outer + (int64_t)kvh * a.stride_head + (int64_t)lo * a.stride_token) * esz;
      const int nrec = hi > lo ? (hi - lo) * row_bytes : 0;
      kc = make_rsrc(static_cast<const char*>(a.k) + base, nrec);
      vc = make_rsrc(static_cast<const char*>(a.v) + base, nrec);
    }
  }

  // Descriptors and SGPR byte offset of key `first` (wave-uniform, >= lo);
  // bad is set when its page is outside the pool.
  __device__ __forceinline__ void at(int first, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv, int& soff,
                                     bool& bad) const {
    if constexpr (kPaged) {
      const int p0 = first & ~15;
      int pid = 0;
      bad = false;
      int nrec = 0;
      if (p0 < hi) {   // never read a block-table entry past the sequence's last page
        pid = a.block_table[(int64_t)b * a.block_table_stride + (p0 >> 4)];
        bad = pid < 0 || pid >= a.num_pages;
        if (bad) pid = 0;
        else nrec = (min(hi, p0 + 16) - p0) * row_bytes;
      }
      const int64_t base = ((int64_t)pid * a.stride_outer + (int64_t)kvh * a.stride_head) * esz;
      rk = make_rsrc(static_cast<const char*>(a.k) + base, nrec);
      rv = make_rsrc(static_cast<const char*>(a.v) + base, nrec);
      soff = (first - p0) * row_bytes;
    } else {
      bad = false;
      rk = kc;
      rv = vc;
      soff = (first - lo) * row_bytes;
    }
  }
};

// Merge the per-wave states (m in base-2 units, l, acc) held in LDS into the
// chunk record: o = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w and
// LSE = ln2 * (M + log2 sum_w 2^(m_w - M) l_w). A chunk with no valid key
// (M = -inf) is written as o = 0, LSE = -inf.
template <int D>
__device__ __forceinline__ void write_record(const PartialLaunch& a, const float* sm_m, const float* sm_l,
                                             const float* sm_acc, int heads, int stride_h, int b, int h0,
                                             int split) {
  const int S = a.num_splits;
  for (int idx = threadIdx.x; idx < heads * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * stride_h + h]);
    const int64_t rec = ((int64_t)b * a.num_q_heads + h0 + h) * S + split;
    float o = 0.0f, lse = neg_inf();
    if (M != neg_inf()) {
      float lsum = 0.0f, osum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm_m[w * stride_h + h] - M);
        lsum += f * sm_l[w * stride_h + h];
        osum += f * sm_acc[(w * stride_h + h) * D + d];
      }
      o = osum / lsum;
      lse = (M + log2f(lsum)) * kLn2;
    }
    a.o_part[rec * D + d] = o;
    if (d == 0) a.lse_part[rec] = lse;
  }
}

// ---------------------------------------------------------------------------
// VALU partial kernel: lanes split head_dim. A key row of D elements is read
// by kLpr lanes with one 16-byte load each, so one wave load covers kRpw
// consecutive rows (1 KiB, contiguous in a [tokens][D] slice). q.k is a
// per-lane partial dot product finished by a DPP sum over the row's lanes;
// p*v accumulates per lane into its own kEpl output elements.
// ---------------------------------------------------------------------------
template <typename T, int D, int GT, bool kPaged>
__global__ __launch_bounds__(kThreads) void partial_valu(PartialLaunch a) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int kEpl = 16 / sizeof(T);   // elements per lane load
  constexpr int kLpr = D / kEpl;         // lanes per key row
  constexpr int kRpw = 64 / kLpr;        // key rows per wave load
  constexpr int kSlots = 8;              // wave loads per tile (each for K and V)
  constexpr int kTile = kSlots * kRpw;   // keys per wave tile
  static_assert(kLpr == 8 || kLpr == 16 || kLpr == 32, "row split");
  static_assert(16 % kRpw == 0 || kRpw % 16 == 0, "page alignment");

  __shared__ float sm_m[kWaves * GT];
  __shared__ float sm_l[kWaves * GT];
  __shared__ float sm_acc[kWaves * GT * D];

  const int split = blockIdx.x;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int tiles_per_kv = group / GT;
  const int kvh = blockIdx.y / tiles_per_kv;
  const int h0 = kvh * group + (blockIdx.y - kvh * tiles_per_kv) * GT;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform for the compiler
  const int row = lane / kLpr;
  const int col = lane - row * kLpr;

  const int L = clamp_len(a, b);
  const int lo = split * a.chunk_len;
  const int hi = min(lo + a.chunk_len, L);

  // This lane's kEpl query elements for each of the GT heads.
  u32x4 qw[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h)
    qw[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.q) +
                                            ((int64_t)b * a.num_q_heads + h0 + h) * D + col * kEpl);

  float m[GT], l[GT], acc[GT][kEpl];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = neg_inf();
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[h][e] = 0.0f;
  }

  struct Tile {
    u32x4 k[kSlots];
    u32x4 v[kSlots];
    uint32_t bad;
  };

  const KvSource<kPaged> src(a, b, kvh, lo, hi, (int)sizeof(T));
  const int voff = row * src.row_bytes + col * 16;

  auto load = [&](Tile& t, int tb) {
    t.bad = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      __amdgpu_buffer_rsrc_t rk, rv;
      int soff;
      bool bad;
      src.at(tb + i * kRpw, rk, rv, soff, bad);
      t.bad |= (uint32_t)bad << i;
      t.k[i] = load16(rk, voff, soff);
      t.v[i] = load16(rv, voff, soff);
    }
  };

  auto dot = [&](const u32x4& q, const u32x4& k) -> float {
    if constexpr (kBf16) {
      float d = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[w]), as_bf16x2(k[w]), d, false);
      return d;
    } else {
      float d = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) d = fmaf(as_f32(q[w]), as_f32(k[w]), d);
      return d;
    }
  };

  auto compute = [&](const Tile& t, int tb) {
    float s[GT][kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const bool valid = (tb + i * kRpw + row < hi) && !((t.bad >> i) & 1u);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float d = group_sum<kLpr>(dot(qw[h], t.k[i]));
        s[h][i] = valid ? d * a.qscale : neg_inf();
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float tm = s[h][0];
#pragma unroll
      for (int i = 1; i < kSlots; ++i) tm = fmaxf(tm, s[h][i]);
      tm = across_max<kLpr>(tm);
      const float mn = fmaxf(m[h], tm);
      if (mn == neg_inf()) continue;   // nothing valid seen yet (wave-uniform)
      if (mn > m[h]) {                 // running max moved: rescale (wave-uniform)
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[h][i] - mn);
        l[h] += p;
        if constexpr (kBf16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[h][2 * w] = fmaf(p, bf16_lo(t.v[i][w]), acc[h][2 * w]);
            acc[h][2 * w + 1] = fmaf(p, bf16_hi(t.v[i][w]), acc[h][2 * w + 1]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] = fmaf(p, as_f32(t.v[i][w]), acc[h][w]);
        }
      }
    }
  };

  // Tiles of this wave: lo + (wave + n * kWaves) * kTile. The next tile is
  // always loaded before the current one is used (with clamped addresses when
  // it lies past hi), so loads stay in flight across the math.
  constexpr int kStep = kWaves * kTile;
  int tb = lo + wave * kTile;
  if (tb < hi) {
    Tile t0, t1;
    load(t0, tb);
    for (;;) {
      load(t1, tb + kStep);
      compute(t0, tb);
      tb += kStep;
      if (tb >= hi) break;
      load(t0, tb + kStep);
      compute(t1, tb);
      tb += kStep;
      if (tb >= hi) break;
    }
  }

  // Finish the wave state: the kRpw rows of the wave hold disjoint keys.
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    l[h] = across_sum<kLpr>(l[h]);
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[h][e] = across_sum<kLpr>(acc[h][e]);
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < kEpl; ++e) sm_acc[(wave * GT + h) * D + col * kEpl + e] = acc[h][e];
      if (col == 0) {
        sm_m[wave * GT + h] = m[h];
        sm_l[wave * GT + h] = l[h];
      }
    }
  }
  __syncthreads();
  write_record<D>(a, sm_m, sm_l, sm_acc, GT, GT, b, h0, split);
}

// ---------------------------------------------------------------------------
// MFMA partial kernel (bf16, head_dim 128, 4 <= g <= 16): the g query heads
// of a KV head form the 16-wide N side of v_mfma_f32_16x16x32_bf16.
//
//   scores  S[key][head] = K_tile(16 keys x 32 dims) * Q^T(32 dims x 16 heads),
//           4 MFMAs over the 128 dims, two 16-key halves per 32-key tile.
//           Lane (G = lane/16, c = lane%16) loads key c of the half, dims
//           32s + 8G .. +8; Q^T is held the same way with c = head.
//   result  lane (G, c) holds the scores of keys 4G + r (r = 0..3) of each
//           half for head c -- exactly the A layout the P*V product needs
//           when key slot (G, e) of the 32-key contraction is key
//           4G + (e % 4) + 16 (e / 4).
//   P*V     O[head][dim] += P(16 heads x 32 keys) * V(32 keys x 16 dims),
//           8 MFMAs; output column c of MFMA j is dim 8c + j, so lane (G, c)
//           loads 16 contiguous bytes (dims 8c .. 8c+7) of each of its 8 keys
//           and transposes them in registers into the 8 B operands.
//   P is rounded to bf16 for the product; the denominator l sums the fp32 P.
// ---------------------------------------------------------------------------
template <bool kPaged>
__global__ __launch_bounds__(kThreads, 2) void partial_mfma_bf16_d128(PartialLaunch a) {
  constexpr int D = 128;
  constexpr int kTile = 32;
  constexpr int kMaxG = 16;
  __shared__ float sm_m[kWaves * kMaxG];
  __shared__ float sm_l[kWaves * kMaxG];
  __shared__ float sm_acc[kWaves * kMaxG * D];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int h0 = kvh * group;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform for the compiler
  const int G = lane >> 4;
  const int c = lane & 15;

  const int L = clamp_len(a, b);
  const int lo = split * a.chunk_len;
  const int hi = min(lo + a.chunk_len, L);

  // Q^T operand: head c (zero past the group), dims 32s + 8G .. +8.
  bf16x8 qop[4];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + h0 + c) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (c < group) w = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * G);
      qop[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  float m = neg_inf();   // running max of head c (base 2), same in the 4 lanes of head c
  float l = 0.0f;        // this lane's share of head c's denominator
  f32x4 acc[8];          // acc[j][r] = O[head 4G + r][dim 8c + j]
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  struct Tile {
    u32x4 k[2][4];
    u32x4 v[8];
    uint32_t bad;
  };
  const KvSource<kPaged> src(a, b, kvh, lo, hi, 2);
  const int voff_k = c * src.row_bytes + 16 * G;       // key c of a 16-key half, dims 32s + 8G
  const int voff_v = 4 * G * src.row_bytes + 16 * c;   // key 4G (+ r via soffset), dims 8c .. 8c+7

  auto load = [&](Tile& t, int tb) {
    t.bad = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      __amdgpu_buffer_rsrc_t rk, rv;
      int soff;
      bool bad;
      src.at(tb + 16 * u, rk, rv, soff, bad);
      t.bad |= (uint32_t)bad << u;
#pragma unroll
      for (int s = 0; s < 4; ++s) t.k[u][s] = load16(rk, voff_k + 64 * s, soff);
#pragma unroll
      for (int r = 0; r < 4; ++r) t.v[4 * u + r] = load16(rv, voff_v, soff + r * src.row_bytes);
    }
  };

  auto compute = [&](const Tile& t, int tb) {
    float s[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[u][st]), qop[st], sc, 0, 0, 0);
      const bool page_ok = !((t.bad >> u) & 1u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = page_ok && (tb + 16 * u + 4 * G + r < hi);
        s[u][r] = valid ? sc[r] * a.qscale : neg_inf();
      }
    }
    float tm = s[0][0];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) tm = fmaxf(tm, s[u][r]);
    tm = across_max<16>(tm);
    const float mn = fmaxf(m, tm);
    const bool live = mn != neg_inf();
    if (__builtin_amdgcn_read_exec() & __ballot(live && mn > m)) {
      // Some head's running max moved: rescale l and that head's accumulators.
      const float alpha = live ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * G + r);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][r] *= ar;
      }
    }
    m = live ? mn : m;
    float p[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[u][r] = live ? __builtin_amdgcn_exp2f(s[u][r] - mn) : 0.0f;
        l += p[u][r];
      }
    bf16x8 pop;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) pop[4 * u + r] = (__bf16)p[u][r];
    // B operand of MFMA j: element e = V[key of slot e][dim 8c + j].
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 w;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const uint32_t x0 = t.v[2 * q2][j >> 1];
        const uint32_t x1 = t.v[2 * q2 + 1][j >> 1];
        w[q2] = (j & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, __builtin_bit_cast(bf16x8, w), acc[j], 0, 0, 0);
    }
  };

  constexpr int kStep = kWaves * kTile;
  int tb = lo + wave * kTile;
  if (tb < hi) {
    Tile t0, t1;
    load(t0, tb);
    for (;;) {
      load(t1, tb + kStep);
      compute(t0, tb);
      tb += kStep;
      if (tb >= hi) break;
      load(t0, tb + kStep);
      compute(t1, tb);
      tb += kStep;
      if (tb >= hi) break;
    }
  }

  const float lt = across_sum<16>(l);   // head c's denominator over the wave
  if (G == 0 && c < group) {
    sm_m[wave * kMaxG + c] = m;
    sm_l[wave * kMaxG + c] = lt;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * G + r;
    if (h < group) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm_acc[(wave * kMaxG + h) * D + 8 * c + j] = acc[j][r];
    }
  }
  __syncthreads();
  write_record<D>(a, sm_m, sm_l, sm_acc, group, kMaxG, b, h0, split);
}

// ---------------------------------------------------------------------------
// Combine. Per (b, h) row: M = max_s LSE_s; w_s = exp(LSE_s - M), zero for an
// empty chunk (LSE = -inf); out = sum_s w_s o_s / sum_s w_s; lse_out = M +
// log(sum_s w_s). A row with only empty chunks gets 0 and -inf.
//
// kWpr waves serve one row. A lane holds 8 consecutive dims (two 16-byte
// loads per record), so D/8 lanes cover a record and the wave's 64/(D/8)
// lane groups, across kWpr waves, take the S records in turn; the partial
// sums are then added across groups (shuffles) and waves (LDS).
// ---------------------------------------------------------------------------
template <typename OutT, int D, int kWpr>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineLaunch a) {
  constexpr int kLanesPerRec = D / 8;
  constexpr int kGroupsPerWave = 64 / kLanesPerRec;
  constexpr int kGroups = kGroupsPerWave * kWpr;
  constexpr int kRowsPerBlock = kWaves / kWpr;
  __shared__ float sm[kWaves][kLanesPerRec][9];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * kRowsPerBlock + wave / kWpr;
  const int wr = wave % kWpr;                       // wave within the row
  const int grp = wr * kGroupsPerWave + lane / kLanesPerRec;
  const int sl = lane % kLanesPerRec;               // dims 8*sl .. 8*sl+7
  const bool live_row = row < a.rows;
  const int S = a.num_splits;
  const float* lse = a.lse_part + (int64_t)(live_row ? row : 0) * S;
  const float* o = a.o_part + (int64_t)(live_row ? row : 0) * S * D + 8 * sl;

  float M = neg_inf();
  if (live_row)
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lse[s]);
  M = across_max<1>(M);
  const bool any = M != neg_inf();

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float wsum = 0.0f;
  if (any) {
    for (int s = grp; s < S; s += kGroups) {
      const float w = expf(lse[s] - M);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(o + (int64_t)s * D);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(o + (int64_t)s * D + 4);
      wsum += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(w, x0[e], acc[e]);
        acc[4 + e] = fmaf(w, x1[e], acc[4 + e]);
      }
    }
  }
  // Lane groups of this wave hold disjoint records of the same dims.
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = across_sum<kLanesPerRec>(acc[e]);
  wsum = across_sum<kLanesPerRec>(wsum);
  if constexpr (kWpr > 1) {
    if (lane < kLanesPerRec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm[wave][sl][e] = acc[e];
      sm[wave][sl][8] = wsum;
    }
    __syncthreads();
    if (wr != 0) return;
    for (int w = 1; w < kWpr; ++w) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += sm[wave + w][sl][e];
      wsum += sm[wave + w][sl][8];
    }
  }
  if (!live_row || lane >= kLanesPerRec) return;
  const int64_t base = (int64_t)row * D + 8 * sl;
  if constexpr (sizeof(OutT) == 2) {
    u32x4 packed;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float r0 = any ? acc[2 * q] / wsum : 0.0f;
      const float r1 = any ? acc[2 * q + 1] / wsum : 0.0f;
      packed[q] = (uint32_t)to_bf16_rne(r0) | ((uint32_t)to_bf16_rne(r1) << 16);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + base) = packed;
  } else {
    f32x4 r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = any ? acc[e] / wsum : 0.0f;
      r1[e] = any ? acc[4 + e] / wsum : 0.0f;
    }
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + base) = r0;
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + base + 4) = r1;
  }
  if (a.lse_out && sl == 0) a.lse_out[row] = any ? M + logf(wsum) : neg_inf();
}

template <typename T, int D, int GT>
hipError_t launch_valu_typed(const PartialLaunch& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  dim3 grid(a.num_splits, a.num_kv_heads * (group / GT), a.batch);
  if (a.paged)
    hipLaunchKernelGGL((partial_valu<T, D, GT, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((partial_valu<T, D, GT, false>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu_d(const PartialLaunch& a, hipStream_t stream) {
  switch (valu_head_tile(a.num_q_heads / a.num_kv_heads)) {
    case 4: return launch_valu_typed<T, D, 4>(a, stream);
    case 2: return launch_valu_typed<T, D, 2>(a, stream);
    default: return launch_valu_typed<T, D, 1>(a, stream);
  }
}

template <typename T>
hipError_t launch_valu(const PartialLaunch& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_valu_d<T, 64>(a, stream) : launch_valu_d<T, 128>(a, stream);
}

template <typename OutT, int D>
hipError_t launch_combine_typed(const CombineLaunch& a, hipStream_t stream) {
  // Waves per row grow with the record count so long split lists are read in
  // parallel: one wave up to 32 records, four from 64.
  const int wpr = a.num_splits >= 64 ? 4 : a.num_splits > 32 ? 2 : 1;
  const int rows_per_block = kWaves / wpr;
  dim3 grid((a.rows + rows_per_block - 1) / rows_per_block);
  if (wpr == 4)
    hipLaunchKernelGGL((combine_kernel<OutT, D, 4>), grid, dim3(kThreads), 0, stream, a);
  else if (wpr == 2)
    hipLaunchKernelGGL((combine_kernel<OutT, D, 2>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<OutT, D, 1>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int valu_head_tile(int group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

bool mfma_supported(int kv_dtype, int head_dim, int group) {
  return kv_dtype == FD_BF16 && head_dim == 128 && group >= 4 && group <= 16;
}

hipError_t launch_partial(const PartialLaunch& a, hipStream_t stream) {
  if (a.path == FD_PATH_MFMA) {
    dim3 grid(a.num_splits, a.num_kv_heads, a.batch);
    if (a.paged)
      hipLaunchKernelGGL(partial_mfma_bf16_d128<true>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(partial_mfma_bf16_d128<false>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (a.kv_dtype == FD_BF16) return launch_valu<uint16_t>(a, stream);
  return launch_valu<float>(a, stream);
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream) {
  if (a.out_dtype == FD_BF16)
    return a.head_dim == 64 ? launch_combine_typed<uint16_t, 64>(a, stream)
                            : launch_combine_typed<uint16_t, 128>(a, stream);
  return a.head_dim == 64 ? launch_combine_typed<float, 64>(a, stream) : launch_combine_typed<float, 128>(a, stream);
}

}  // namespace fd
