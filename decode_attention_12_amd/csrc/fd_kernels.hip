// fd_kernels.hip -- gfx950 kernels for split-KV decode attention.
//
// Pages cited (by title and section):
//   [QA]    "FlashDecoding面经-vivj啥关系 vi就是原来的O呗用LSE是为了防止溢出吗",
//           parts 二 (a chunk writes acc_i / l_i, its locally normalised
//           output) and 三 (LSE_i = m_i + log l_i; weights exp(LSE_i - max)).
//   [MERGE] www.2kiu.com/news/6053916, "用 log-sum-exp 给块结果定权重" (an empty
//           chunk must not become a zero output with normal weight) and
//           "分块数量是一笔成本账" (masks consistent across chunks; paged
//           logical order; the chunk count is a cost trade-off, and the
//           schedule should follow batch and context).
//   [INFRA] "AI Infra：深入理解大模型中的数学与Infra优化", 2.3 (subtract the
//           max), 2.4 (scale), 2.5 (masked keys leave numerator and
//           denominator; block-table gather), 2.6 (online softmax: running
//           max, rescale by exp(m_old - m_new), the (m, l, O) state; "LSE 与
//           Online Softmax": P = exp2 after one FMA; "Flash-Decoding 的
//           Split-K": each chunk writes its local O and LSE, a reduction
//           kernel merges them; the FA3 note on persistent workers pulling
//           their own work).
//
// A partial kernel is a per-wave engine (the online-softmax state of a run
// of one KV head's query rows, plus the tile load and tile math) under one
// of two drivers:
//
//   split mode     one workgroup of four waves per (split, segment,
//                  sequence); the waves take the chunk's tiles in turn and
//                  merge their four states through LDS into one record.
//   balanced mode  persistent worker waves. The key tiles (16 .. 128 keys) of
//                  every (sequence, segment) are laid end to end and cut into
//                  equal runs, one per worker, whatever the sequence lengths;
//                  a worker streams its run with loads for the next tile
//                  (across segment boundaries) in flight, and writes one
//                  record per segment piece. The piece of segment s done by
//                  worker p goes to record slot s + p, so each segment's
//                  records are one contiguous run of slots.
//
// Each K/V byte is fetched once per segment: a segment holds every query row
// that reads its KV head when they fit one matrix tile (the MFMA engine), or
// a tile of 1, 2 or 4 of them (the VALU engine).
//
// Scores are kept in base-2 units: q.k is multiplied by scale*log2(e), so the
// exponentials are single v_exp_f32 (2^x) instructions; the LSE of a record
// is converted back to the natural log when it is written.
//
// Query rows: a sequence has q_len * Hq of them, token-major (row (t, h) is
// t * Hq + h). The rows that read KV head kvh are its q_len * g rows
// (t, kvh * g + i), taken in (t, i) order; a segment holds a run of R of them
// (R = rows_per_seg). Token t of q_len sees keys [0, L_b - q_len + 1 + t)
// ([INFRA] 2.5: the causal rule, which multi-token verification needs).
//
// fp8 (E4M3) caches: K/V bytes are converted to bf16 in registers (exact:
// every E4M3 value is a bf16 value) and fed to the same dot products; the
// per-KV-head scales are applied once per segment -- the key scale folded
// into the score multiplier, the value scale into the record's 1/l.
//
// Masking: a key at or past the row's limit (end of the chunk, L_b, or the
// token's window), or on a page whose block-table entry is outside the pool,
// gets score -inf and so weight 0.
// K/V come in through buffer loads over 16-key groups whose range ends at key
// hi, so such keys read as zeros (never NaN into p*v), no load leaves the
// valid part of the cache, and block-table entries past the sequence's last
// page are never read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "fd_internal.h"

// The workspace of fd_decode_static: a device array of fixed size that the
// library owns, for callers that cannot allocate. Each GPU the library runs
// on holds its own copy (at its own address) until the process ends. In host
// code this name stands for the array but is not its device address; host
// code uses the address hipGetSymbolAddress gives (static_workspace below).
static __device__ __align__(256) char scratch[fd::kStaticWorkspaceBytes];

namespace fd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Kernel template modes: the fd_mode values plus the single-launch balanced variant.
constexpr int kModeBalancedFused = 2;
constexpr float kLn2 = 0.69314718055994530942f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

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

// E4M3 -> bf16 / fp32 conversion of the two bytes in the low (kHi = false)
// or high half of w; the lower byte becomes element 0. Scale operand 1.0:
// no rescaling in the conversion.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}
template <bool kHi>
__device__ __forceinline__ f32x2 e4m3x2_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, kHi);
}

// Key/value storage: float (fp32), uint16_t (bf16) or uint8_t (fp8 E4M3).
template <typename KV>
struct KvType {
  static constexpr int kBytes = sizeof(KV);
  static constexpr bool kF32 = sizeof(KV) == 4;
  static constexpr bool kFp8 = sizeof(KV) == 1;
  static constexpr int kQBytes = kF32 ? 4 : 2;   // q is bf16 unless the cache is fp32
};

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
  static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16 || kLanes == 32, "group size");
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if constexpr (kLanes == 4) {
  } else if constexpr (kLanes == 8) {
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

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Wave index that the compiler knows to be wave-uniform, so offsets and
// descriptors derived from it stay in SGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Read-only int32 tables (sequence lengths, block table) at wave-uniform
// indices. Going through the constant address space makes these scalar loads:
// as vector loads, the wait for their value would also wait for every K/V
// load in flight.
__device__ __forceinline__ int load_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

__device__ __forceinline__ float load_uniform_f(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}

__device__ __forceinline__ int clamp_len(const PartialLaunch& a, int b) {
  const int L = load_uniform(a.seq_lens, b);
  return min(max(L, 0), a.max_seq_len);
}

// Output (and q) row of row c of KV head kvh's q_len * g rows in sequence b.
template <class Launch>
__device__ __forceinline__ int64_t out_row(const Launch& a, int b, int kvh, int c) {
  const int g = a.num_q_heads / a.num_kv_heads;
  const int t = c / g;
  return ((int64_t)b * a.geo.q_len + t) * a.num_q_heads + kvh * g + (c - t * g);
}

// Keys row c of a segment may use: those below the piece end hi and inside
// its token's window, [0, len - q_len + 1 + t).
__device__ __forceinline__ int row_limit(const PartialLaunch& a, int c, int hi, int len) {
  const int g = a.num_q_heads / a.num_kv_heads;
  return min(hi, len - a.geo.q_len + 1 + c / g);
}

// Per-segment scales: the score multiplier (scale * log2 e, times the key
// scale of an fp8 cache) and the value scale.
template <bool kFp8>
__device__ __forceinline__ void segment_scales(const PartialLaunch& a, int kvh, float& qs, float& vs) {
  if constexpr (kFp8) {
    qs = a.qscale * load_uniform_f(a.k_scale, kvh);
    vs = load_uniform_f(a.v_scale, kvh);
  } else {
    qs = a.qscale;
    vs = 1.0f;
  }
}

// ---------------------------------------------------------------------------
// K/V source: buffer descriptors over 16-key groups of one (sequence, KV
// head). A group is a page of a paged cache, or 16 consecutive rows of a
// contiguous one; its descriptor covers only the rows below hi.
// ---------------------------------------------------------------------------
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer, gfx9-family descriptor word 3
constexpr int kStreamLoad = 2;             // nontemporal: every K/V byte is read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_records, kBufferWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, kStreamLoad));
}
__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voffset, soffset, kStreamLoad));
}

template <bool kPaged>
struct KvSource {
  const char* kbase;      // contiguous: row 0 of the (b, kvh) slice; paged: pool + kvh * stride_head
  const char* vbase;
  const int32_t* table;   // paged: block-table row of the sequence
  int64_t page_bytes;     // paged: stride_outer in bytes
  int num_pages;
  int page_shift;         // paged: log2 of the page size (a power of two, 16 .. 256)
  int hi;                 // rows at or past hi read as zeros
  int row_bytes;

  __device__ __forceinline__ void init(const PartialLaunch& a, int b, int kvh, int hi_, int esz) {
    hi = hi_;
    row_bytes = (int)a.stride_token * esz;
    num_pages = a.num_pages;
    page_shift = a.page_shift;
    page_bytes = a.stride_outer * esz;
    if constexpr (kPaged) {
      const int64_t off = a.stride_head * kvh * esz;
      kbase = static_cast<const char*>(a.k) + off;
      vbase = static_cast<const char*>(a.v) + off;
      table = a.block_table + (int64_t)b * a.block_table_stride;
    } else {
      const int64_t off = (a.stride_outer * b + a.stride_head * kvh) * esz;
      kbase = static_cast<const char*>(a.k) + off;
      vbase = static_cast<const char*>(a.v) + off;
      table = nullptr;
    }
  }

  // Nothing to read: every descriptor comes out empty.
  __device__ __forceinline__ void none() { hi = 0; }

  // Descriptors of the 16-key group holding key `first` (wave-uniform), the
  // SGPR byte offset of `first` inside it, and whether its page is outside
  // the pool. Pages hold a multiple of 16 keys, so a group never straddles
  // two pages.
  __device__ __forceinline__ void at(int first, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv, int& soff,
                                     bool& bad) const {
    const int g0 = first & ~15;
    int nrec = 0;
    bad = false;
    const char* kb = kbase;
    const char* vb = vbase;
    if (g0 < hi) {
      nrec = min(hi - g0, 16) * row_bytes;
      if constexpr (kPaged) {
        int pid = load_uniform(table, g0 >> page_shift);
        bad = pid < 0 || pid >= num_pages;
        if (bad) {
          nrec = 0;
          pid = 0;
        }
        const int64_t in_page = (int64_t)(g0 & ((1 << page_shift) - 1)) * row_bytes;
        kb += page_bytes * pid + in_page;
        vb += page_bytes * pid + in_page;
      } else {
        kb += (int64_t)g0 * row_bytes;
        vb += (int64_t)g0 * row_bytes;
      }
    }
    rk = make_rsrc(kb, nrec);
    rv = make_rsrc(vb, nrec);
    soff = (first - g0) * row_bytes;
  }
};

// Record stores. The single-launch variant writes records with agent-scope
// coherent stores (sc1: written through past this XCD's L2), so that another
// XCD's wave can read them without a cache-wide writeback or invalidate.
// Vectors go out as 16-byte buffer stores with that cache policy: lanes that
// each wrote 4 floats as 4 separate dword stores left partial lines to be
// written through one by one.
constexpr int kCoherentPolicy = 16;   // sc1, as the agent-scope atomic loads and stores use
constexpr int kWholeRange = 0x7fffffff;

__device__ __forceinline__ void put1(float* p, float v, bool coherent) {
  if (coherent)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
// Four floats at base + byte_off; base is wave-uniform.
__device__ __forceinline__ void put4(float* base, int byte_off, f32x4 v, bool coherent) {
  if (coherent)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), make_rsrc(base, kWholeRange), byte_off, 0,
                                           kCoherentPolicy);
  else
    *reinterpret_cast<f32x4*>(reinterpret_cast<char*>(base) + byte_off) = v;
}

// A record's LSE in natural-log units, ln2 * (m + log2 l), from the base-2
// running max m and sum l; -inf when the piece saw no valid key (its output
// is then written as 0).
__device__ __forceinline__ float record_lse(float m, float l) {
  return m == neg_inf() ? neg_inf() : (m + log2f(l)) * kLn2;
}

// Merge four waves' states held in LDS into split-mode records:
// o = vs * sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w, LSE = ln2 (M +
// log2 of that denominator); a chunk with no valid key gets o = 0,
// LSE = -inf. The records are those of rows c0 .. c0 + rows - 1 of KV head
// kvh. A thread writes 4 consecutive dims with one 16-byte store.
template <int D>
__device__ __forceinline__ void merge_waves(const PartialLaunch& a, const float* sm_m, const float* sm_l,
                                            const float* sm_acc, int rows, int stride_h, int b, int kvh, int c0,
                                            int split, float vs) {
  const int S = a.geo.num_splits;
  const bool coherent = a.out != nullptr;
  const int64_t row0 = out_row(a, b, kvh, c0);
  float* base = a.o_part + (row0 * S + split) * D;   // wave-uniform
  for (int idx = threadIdx.x; idx < rows * (D / 4); idx += kThreads) {
    const int h = idx / (D / 4);
    const int d0 = 4 * (idx - h * (D / 4));
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * stride_h + h]);
    const int64_t drow = out_row(a, b, kvh, c0 + h) - row0;   // within q_len * Hq rows
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    float lse = neg_inf();
    if (M != neg_inf()) {
      float lsum = 0.0f;
      f32x4 osum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm_m[w * stride_h + h] - M);
        lsum += f * sm_l[w * stride_h + h];
        const float* src = sm_acc + (w * stride_h + h) * D + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) osum[e] += f * src[e];
      }
      const float inv = vs / lsum;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = osum[e] * inv;
      lse = record_lse(M, lsum);
    }
    const int64_t eoff = drow * S * D + d0;
    if (coherent)
      put4(base, (int)(eoff * 4), o, true);   // the single launch keeps records below 2^31 bytes
    else
      *reinterpret_cast<f32x4*>(base + eoff) = o;
    if (d0 == 0) put1(a.lse_part + (row0 + drow) * S + split, lse, coherent);
  }
}

// Final outputs in out_dtype: one element, or N (4, 8 or 16) consecutive
// elements from idx, a multiple of N, with 8- or 16-byte stores.
__device__ __forceinline__ void store_out(const PartialLaunch& a, int64_t idx, float v) {
  if (a.out_dtype == FD_BF16)
    reinterpret_cast<uint16_t*>(a.out)[idx] = to_bf16_rne(v);
  else
    reinterpret_cast<float*>(a.out)[idx] = v;
}

template <int N>
__device__ __forceinline__ void store_out_vec(const PartialLaunch& a, int64_t idx, const float* v) {
  static_assert(N % 4 == 0, "whole groups of four");
  if (a.out_dtype == FD_BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + idx;
#pragma unroll
    for (int q0 = 0; q0 < N; q0 += 4) {
      const u32x2 w = {(uint32_t)to_bf16_rne(v[q0]) | ((uint32_t)to_bf16_rne(v[q0 + 1]) << 16),
                       (uint32_t)to_bf16_rne(v[q0 + 2]) | ((uint32_t)to_bf16_rne(v[q0 + 3]) << 16)};
      *reinterpret_cast<u32x2*>(o + q0) = w;
    }
  } else {
    float* o = reinterpret_cast<float*>(a.out) + idx;
#pragma unroll
    for (int q0 = 0; q0 < N; q0 += 4) *reinterpret_cast<f32x4*>(o + q0) = f32x4{v[q0], v[q0 + 1], v[q0 + 2], v[q0 + 3]};
  }
}

// ---------------------------------------------------------------------------
// VALU engine: lanes split head_dim. A key row of D elements is read by kLpr
// lanes with one 16-byte load each, so one wave load covers kRpw consecutive
// rows. q.k is a per-lane partial dot product (v_dot2c_f32_bf16 on bf16 pairs,
// fp8 bytes converted to bf16 pairs first, or FMA for fp32) finished by a DPP
// sum over the row's lanes; p*v accumulates per lane into its own kEpl output
// elements. Handles GT query rows of one KV head.
// ---------------------------------------------------------------------------
template <typename KV, int D, int GT, bool kPaged>
struct ValuEngine {
  using Ty = KvType<KV>;
  static constexpr int kEsz = Ty::kBytes;
  static constexpr int kEpl = 16 / kEsz;       // KV elements per lane load
  static constexpr int kQl = kEpl * Ty::kQBytes / 16;   // 16-byte q loads per lane and row
  static constexpr int kLpr = D / kEpl;        // lanes per key row
  static constexpr int kRpw = 64 / kLpr;       // key rows per wave load
  static constexpr int kSlots = 8;             // wave loads per tile (each for K and V)
  static constexpr int kStageBytes = 0;        // no LDS K stage
  static constexpr int kTailUnroll = 8;        // records per lane in flight in the single-launch split tail
  static constexpr int kLoadsPerTile = 2 * kSlots;
  static constexpr int kTile = kSlots * kRpw;  // keys per wave tile: 16 .. 128
  static constexpr int kGroups = kTile / 16;   // 16-key groups per tile
  static constexpr int kSlotsPerGroup = kSlots / kGroups;
  static constexpr int kD = D;
  static_assert(kLpr == 4 || kLpr == 8 || kLpr == 16 || kLpr == 32, "row split");
  static_assert(kTile % 16 == 0 && kSlots % kGroups == 0, "tiles cover whole 16-key groups");
  using Source = KvSource<kPaged>;

  struct Tile {
    u32x4 k[kSlots];
    u32x4 v[kSlots];
    uint32_t bad;
    int buf;              // unused here: the tile's K lives in registers
  };

  int row, col, voff;
  u32x4 q[GT][kQl];
  float m[GT], l[GT], acc[GT][kEpl];
  int lim[GT];          // keys [0, lim) are visible to row h of the segment
  float qs, vs;         // score multiplier and value scale of the segment

  __device__ __forceinline__ void init(const PartialLaunch& a, int lane) {
    row = lane / kLpr;
    col = lane - row * kLpr;
    voff = row * (int)a.stride_token * kEsz + col * 16;
  }

  // Load this lane's kEpl query elements of rows c0 .. c0+GT-1 of KV head
  // kvh in sequence b into q (only where q is dead: before a piece's first
  // tile is computed).
  __device__ __forceinline__ void fetch_q(const PartialLaunch& a, int b, int kvh, int c0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const char* qrow = static_cast<const char*>(a.q) + (out_row(a, b, kvh, c0 + h) * D + col * kEpl) * Ty::kQBytes;
#pragma unroll
      for (int w = 0; w < kQl; ++w) q[h][w] = *reinterpret_cast<const u32x4*>(qrow + 16 * w);
    }
  }

  // Rows c0 .. c0+GT-1 of KV head kvh over a piece ending at key hi of a
  // sequence of len keys.
  __device__ __forceinline__ void window(const PartialLaunch& a, int kvh, int c0, int hi, int len) {
#pragma unroll
    for (int h = 0; h < GT; ++h) lim[h] = row_limit(a, c0 + h, hi, len);
    segment_scales<Ty::kFp8>(a, kvh, qs, vs);
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      m[h] = neg_inf();
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < kEpl; ++e) acc[h][e] = 0.0f;
    }
  }

  // Load order. With 16-bit (and fp32) elements all of the tile's K loads go
  // out before its V loads (the scheduling barrier keeps them apart); with
  // fp8 each K load is followed by the V load of the same rows. Measured on
  // MI355X (A/B rounds on one box, two boxes): K first is 0.1-0.6 % faster
  // on long-context MHA in bf16 and 1.5 % slower with the fp8 cache.
  static constexpr bool kKFirst = kEsz >= 2;

  __device__ __forceinline__ void load(Tile& t, const Source& src, int tb) const {
    t.bad = 0;
    __amdgpu_buffer_rsrc_t rvs[kGroups];
    int soffs[kGroups];
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      __amdgpu_buffer_rsrc_t rk;
      bool bad;
      src.at(tb + 16 * gi, rk, rvs[gi], soffs[gi], bad);
      if (bad) t.bad |= ((1u << kSlotsPerGroup) - 1u) << (gi * kSlotsPerGroup);
#pragma unroll
      for (int si = 0; si < kSlotsPerGroup; ++si) {
        const int i = gi * kSlotsPerGroup + si;
        const int so = soffs[gi] + si * kRpw * src.row_bytes;
        t.k[i] = load16(rk, voff, so);
        if constexpr (!kKFirst) t.v[i] = load16(rvs[gi], voff, so);
      }
    }
    if constexpr (kKFirst) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) {
#pragma unroll
        for (int si = 0; si < kSlotsPerGroup; ++si)
          t.v[gi * kSlotsPerGroup + si] = load16(rvs[gi], voff, soffs[gi] + si * kRpw * src.row_bytes);
      }
    }
  }

  // This lane's partial q.k of row h with one key load (bf16 pairs for fp8:
  // kb holds the converted key, word w = elements 2w, 2w+1).
  __device__ __forceinline__ float dot(int h, const u32x4& kv, const uint32_t* kb) const {
    float d = 0.0f;
    if constexpr (Ty::kF32) {
#pragma unroll
      for (int w = 0; w < 4; ++w) d = fmaf(as_f32(q[h][0][w]), as_f32(kv[w]), d);
    } else if constexpr (Ty::kFp8) {
#pragma unroll
      for (int w = 0; w < 8; ++w)
        d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[h][w >> 2][w & 3]), as_bf16x2(kb[w]), d, false);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[h][0][w]), as_bf16x2(kv[w]), d, false);
    }
    return d;
  }

  // Online-softmax update with the keys [tb, tb + kTile) of the tile; keys
  // at or past a row's limit, or on a bad page, are masked for it.
  __device__ __forceinline__ void compute(const Tile& t, int tb) {
    float s[GT][kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int key = tb + i * kRpw + row;
      const bool page_ok = !((t.bad >> i) & 1u);
      uint32_t kb[8];
      if constexpr (Ty::kFp8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kb[2 * w] = e4m3x2_bf16x2<false>(t.k[i][w]);
          kb[2 * w + 1] = e4m3x2_bf16x2<true>(t.k[i][w]);
        }
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float d = group_sum<kLpr>(dot(h, t.k[i], kb));
        s[h][i] = (page_ok && key < lim[h]) ? d * qs : neg_inf();
      }
    }
    if constexpr (Ty::kFp8) {
      // Rescale every row first, then walk the slots once, converting each
      // value load a single time for all rows.
      float mrow[GT];
      bool live[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float tm = s[h][0];
#pragma unroll
        for (int i = 1; i < kSlots; ++i) tm = fmaxf(tm, s[h][i]);
        tm = across_max<kLpr>(tm);
        const float mn = fmaxf(m[h], tm);
        live[h] = mn != neg_inf();     // wave-uniform
        if (live[h] && mn > m[h]) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < kEpl; ++e) acc[h][e] *= alpha;
          m[h] = mn;
        }
        mrow[h] = mn;
      }
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        float vf[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2 lo = e4m3x2_f32x2<false>(t.v[i][w]);
          const f32x2 hi = e4m3x2_f32x2<true>(t.v[i][w]);
          vf[4 * w] = lo[0];
          vf[4 * w + 1] = lo[1];
          vf[4 * w + 2] = hi[0];
          vf[4 * w + 3] = hi[1];
        }
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          if (!live[h]) continue;
          const float p = __builtin_amdgcn_exp2f(s[h][i] - mrow[h]);
          l[h] += p;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
      return;
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
        if constexpr (Ty::kF32) {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] = fmaf(p, as_f32(t.v[i][w]), acc[h][w]);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[h][2 * w] = fmaf(p, bf16_lo(t.v[i][w]), acc[h][2 * w]);
            acc[h][2 * w + 1] = fmaf(p, bf16_hi(t.v[i][w]), acc[h][2 * w + 1]);
          }
        }
      }
    }
  }

  // The kRpw rows of a wave hold disjoint keys: add them up.
  __device__ __forceinline__ void finish_rows() {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      l[h] = across_sum<kLpr>(l[h]);
#pragma unroll
      for (int e = 0; e < kEpl; ++e) acc[h][e] = across_sum<kLpr>(acc[h][e]);
    }
  }

  __device__ __forceinline__ void to_lds(float* sm_m, float* sm_l, float* sm_acc, int wave) {
    finish_rows();
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
  }

  // Balanced mode: this wave's piece of a segment is a complete record.
  template <bool kCoherent>
  __device__ __forceinline__ void to_record(const PartialLaunch& a, int slot) {
    finish_rows();
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float inv = m[h] == neg_inf() ? 0.0f : vs / l[h];
        float* rec = a.o_part + (int64_t)slot * GT * D;
#pragma unroll
        for (int e = 0; e < kEpl; e += 4)
          put4(rec, (h * D + col * kEpl + e) * 4,
               f32x4{acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv, acc[h][e + 3] * inv}, kCoherent);
        if (col == 0) put1(a.lse_part + (int64_t)slot * GT + h, record_lse(m[h], l[h]), kCoherent);
      }
    }
  }

  // Single launch, a piece that is its whole segment: the record is already
  // the result, so write it as the final rows c0.. of KV head kvh in b.
  __device__ __forceinline__ void to_output(const PartialLaunch& a, int b, int kvh, int c0) {
    finish_rows();
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float inv = m[h] == neg_inf() ? 0.0f : vs / l[h];
        const int64_t orow = out_row(a, b, kvh, c0 + h);
        float o[kEpl];
#pragma unroll
        for (int e = 0; e < kEpl; ++e) o[e] = acc[h][e] * inv;
        store_out_vec<kEpl>(a, orow * D + col * kEpl, o);
        if (a.lse_out && col == 0) a.lse_out[orow] = record_lse(m[h], l[h]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA engine (bf16 or fp8 KV, head_dim 128, 4 .. 16 query rows): the rows
// of a segment form the 16-wide N side of v_mfma_f32_16x16x32_bf16.
//
//   scores  S[key][row] = K_tile(16 keys x 32 dims) * Q^T(32 dims x 16 rows),
//           4 MFMAs over the 128 dims, two 16-key halves per 32-key tile.
//           Lane (G = lane/16, c = lane%16) feeds key c of the half to MFMA
//           st with 8 of its dims: bf16 -- dims 32st + 8G .. +8, one 16-byte
//           load per MFMA; fp8 -- dims 64p + 16G + 8e .. +8 for st = 2p + e,
//           so that one 16-byte load (dims 64p + 16G .. +16) feeds two MFMAs
//           after conversion. Q^T is held the same way with c = row; the
//           contraction does not care which dims an MFMA sums, only that Q
//           and K agree.
//   result  lane (G, c) holds the scores of keys 4G + r (r = 0..3) of each
//           half for row c -- exactly the A layout the P*V product needs
//           when key slot (G, e) of the 32-key contraction is key
//           4G + (e % 4) + 16 (e / 4).
//   P*V     O[row][dim] += P(16 rows x 32 keys) * V(32 keys x 16 dims),
//           8 MFMAs; output column c of MFMA j is dim 8c + j, so lane (G, c)
//           loads dims 8c .. 8c+7 of each of its 8 keys (16 bytes bf16, 8
//           bytes fp8, converted to bf16) and transposes them in registers
//           into the 8 B operands.
//   P enters the product as two bf16 tiles, bf16(p) and bf16(p - bf16(p)),
//   so the weights keep ~17 bits; the denominator l sums the fp32 P.
//   fp8 K   that operand layout puts 16 keys x 64 bytes under one wave load
//           (half of each 128-byte fp8 row), which streams slower from HBM
//           than whole rows. The fp8 kernel therefore copies whole rows of K
//           (8 rows of 16-byte chunks per wave load) straight into LDS with
//           buffer loads (keys past the piece end land as zeros), chunk q of
//           row r at chunk q ^ ((r >> 1) & 7), and reads each operand back
//           with one ds_read_b128, the swizzle keeping a read's 16 lanes on
//           distinct banks. Two tile buffers per wave. (For bf16 the same
//           staging measured within 2 % of loading K into registers, either
//           way depending on the shape, so the bf16 kernel keeps the
//           register path.)
// ---------------------------------------------------------------------------
template <bool kC, typename A, typename B>
struct Pick { using T = A; };
template <typename A, typename B>
struct Pick<false, A, B> { using T = B; };

// s_waitcnt simm16 (gfx9) that waits until at most n vector memory
// operations are outstanding: vmcnt in bits 3:0 and 15:14, expcnt (6:4) and
// lgkmcnt (11:8) left at their maxima.
constexpr int vmcnt_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <bool kPaged, bool kFp8>
struct MfmaEngine {
  static constexpr int D = 128;
  static constexpr int kD = D;
  static constexpr int kTile = 32;
  static constexpr int kMaxRows = 16;
  static constexpr int kEsz = kFp8 ? 1 : 2;
  static constexpr bool kLdsK = kFp8;                     // K through LDS (see above)
  static_assert(kLdsK || !kFp8, "the fp8 operand is read from LDS");
  static constexpr int kKLoads = kFp8 ? 2 : 4;          // wave loads of K per 16-key half
  static constexpr int kVLoads = 4;                       // wave loads of V per 16-key half
  static constexpr int kLoadsPerHalf = kKLoads + kVLoads;
  static constexpr int kLoadsPerTile = 2 * kLoadsPerHalf; // vector memory operations load() issues
  static constexpr int kRowBytes = D * kEsz;              // LDS K stage: one key row
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 64 / kChunks;       // rows one wave load copies
  static constexpr int kHalfBytes = 16 * kRowBytes;
  // A wave load moves 64 lanes x 16 bytes: the K loads of a half cover its
  // 16 rows (LDS copies of whole rows, or register operands of 16 rows x 64
  // bytes), and lane (G, c) loads V for keys 4G .. 4G + 3 of the half, one
  // key per V load.
  static_assert(kKLoads * 64 * 16 == kHalfBytes, "K loads cover the half");
  static_assert(kVLoads * 4 == 16, "V loads cover the half");
  static constexpr int kStageBytes = kLdsK ? 2 * 2 * kHalfBytes : 0;   // per wave: two tiles of two halves
  static constexpr int kTailUnroll = 16;   // the split tail fits in the registers the main loop needs anyway
  using VLoad = typename Pick<kFp8, u32x2, u32x4>::T;
  using Source = KvSource<kPaged>;

  struct Tile {
    u32x4 k[2][kLdsK ? 1 : kKLoads];   // register K (bf16)
    VLoad v[8];
    uint32_t bad;
    int buf;                          // LDS K: which of the wave's two tile buffers
  };

  // LDS K: chunk slot of chunk q of row r is q ^ swizzle(r), so that the 16
  // lanes of a read (16 rows, one chunk each) fall on distinct banks.
  static __device__ __forceinline__ int swizzle(int r) { return kFp8 ? (r >> 1) & 7 : r & 15; }

  int G, c, rows, voff_v, row_bytes;
  int voff_k[kLdsK ? kKLoads : 1];   // register K: key c, dims 8G..; LDS K: this lane's chunk of wave load i
  lds_char* kst;                     // LDS K: this wave's stage [2 tiles][2 halves][16 rows][kRowBytes]
  int lim;              // keys [0, lim) are visible to row c of the segment
  float qs, vs;         // score multiplier and value scale of the segment
  bf16x8 q[4];          // Q^T operand of MFMA st: row c, 8 dims (see above)
  float m;              // running max of row c (base 2), same in the 4 lanes of row c
  float l;              // this lane's share of row c's denominator
  f32x4 acc[8];         // acc[j][r] = O[row 4G + r][dim 8c + j]

  __device__ __forceinline__ void init(const PartialLaunch& a, int lane) {
    G = lane >> 4;
    c = lane & 15;
    rows = a.geo.rows_per_seg;
    row_bytes = (int)a.stride_token * kEsz;
    if constexpr (kLdsK) {
      // Wave load i copies rows kRowsPerLoad * i + lane / kChunks; this
      // lane's chunk slot j holds chunk j ^ swizzle(row) of its row.
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {
        const int r = kRowsPerLoad * i + lane / kChunks;
        voff_k[i] = r * row_bytes + 16 * ((lane % kChunks) ^ swizzle(r));
      }
    } else {
      voff_k[0] = c * row_bytes + 16 * G;                     // key c of a 16-key half
    }
    voff_v = 4 * G * row_bytes + (kFp8 ? 8 : 16) * c;         // key 4G (+ r via soffset), dims 8c .. 8c+7
  }

  // Load the Q^T operand of rows c0.. of KV head kvh in sequence b into q,
  // only where q is dead (before a piece's first tile is computed). Lanes
  // past the segment's rows load a real row again; their score columns are
  // masked and never written. These are ordinary loads into registers, so
  // the compiler keeps exact waits for the K/V loads around them; copying
  // the rows through LDS (global-to-LDS loads) made it turn every later K/V
  // wait into a full drain, prefetched tile included.
  __device__ __forceinline__ void fetch_q(const PartialLaunch& a, int b, int kvh, int c0) {
    const int rc = c < rows ? c : c % rows;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + out_row(a, b, kvh, c0 + rc) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = kFp8 ? 64 * (s >> 1) + 16 * G + 8 * (s & 1) : 32 * s + 8 * G;
      q[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + d0));
    }
  }

  __device__ __forceinline__ void window(const PartialLaunch& a, int kvh, int c0, int hi, int len) {
    lim = c < rows ? row_limit(a, c0 + c, hi, len) : 0;
    segment_scales<kFp8>(a, kvh, qs, vs);
  }

  __device__ __forceinline__ void reset() {
    m = neg_inf();
    l = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  __device__ __forceinline__ lds_char* k_half(int buf, int u) const { return kst + (2 * buf + u) * kHalfBytes; }

  // Issues exactly kLoadsPerTile vector memory operations, in this order:
  // half 0's kKLoads K loads, its kVLoads V loads, then half 1's. The
  // scheduling barriers keep that order (wait_k counts on it).
  __device__ __forceinline__ void load(Tile& t, const Source& src, int tb) const {
    t.bad = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      __amdgpu_buffer_rsrc_t rk, rv;
      int soff;
      bool bad;
      src.at(tb + 16 * u, rk, rv, soff, bad);
      t.bad |= (uint32_t)bad << u;
      if constexpr (kLdsK) __builtin_amdgcn_sched_barrier(0);
      if constexpr (kLdsK) {
        lds_char* dst = k_half(t.buf, u);
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + 1024 * i), 16, voff_k[i], soff, 0,
                                                   kStreamLoad);
      } else {
#pragma unroll
        for (int s = 0; s < kKLoads; ++s) t.k[u][s] = load16(rk, voff_k[0], soff + 64 * s);
      }
      if constexpr (kLdsK) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < kVLoads; ++r) {
        if constexpr (kFp8)
          t.v[4 * u + r] = load8(rv, voff_v, soff + r * row_bytes);
        else
          t.v[4 * u + r] = load16(rv, voff_v, soff + r * row_bytes);
      }
    }
    if constexpr (kLdsK) __builtin_amdgcn_sched_barrier(0);
  }

  // LDS K: wait until half u of a tile has landed (the compiler does not
  // track LDS written by buffer-to-LDS loads). Vector memory operations
  // complete in issue order, and the drivers issue the next tile's load()
  // before computing this one; so after half u's last K load there were
  // issued at least: its kVLoads V loads, half 1's kLoadsPerHalf loads when
  // u = 0, and the next tile's kLoadsPerTile. Waiting until at most that many
  // are outstanding means half u's K has landed. Other operations issued in
  // between (a new piece's query loads, a closed piece's record stores) only
  // make that wait longer than needed, never too short.
  template <int u>
  static constexpr int kKWaitCount = kVLoads + (1 - u) * kLoadsPerHalf + kLoadsPerTile;
  static_assert(kKWaitCount<0> < 64 && kKWaitCount<1> < kKWaitCount<0>, "vmcnt holds 6 bits");
  template <int u>
  __device__ __forceinline__ void wait_k() const {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(kKWaitCount<u>));
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }

  // LDS K: chunk q of key c of half u.
  __device__ __forceinline__ u32x4 k_chunk(const Tile& t, int u, int q) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(k_half(t.buf, u) + c * kRowBytes +
                                                                             16 * (q ^ swizzle(c)));
  }

  // A operand of score MFMA st for half u.
  __device__ __forceinline__ bf16x8 k_operand(const Tile& t, int u, int st) const {
    if constexpr (kFp8) {
      // Chunk q = 4p + G of key c holds dims 64p + 16G .. +16 (st = 2p + e).
      const u32x4 w = k_chunk(t, u, 4 * (st >> 1) + G);
      const int e = st & 1;
      const u32x4 x = {e4m3x2_bf16x2<false>(w[2 * e]), e4m3x2_bf16x2<true>(w[2 * e]),
                       e4m3x2_bf16x2<false>(w[2 * e + 1]), e4m3x2_bf16x2<true>(w[2 * e + 1])};
      return __builtin_bit_cast(bf16x8, x);
    } else if constexpr (kLdsK) {
      return __builtin_bit_cast(bf16x8, k_chunk(t, u, 4 * st + G));   // dims 32st + 8G .. +8
    } else {
      return __builtin_bit_cast(bf16x8, t.k[u][st]);
    }
  }

  __device__ __forceinline__ void compute(const Tile& t, int tb) {
    float s[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (kLdsK) {
        if (u == 0) wait_k<0>();
        else wait_k<1>();
      }
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < 4; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(t, u, st), q[st], sc, 0, 0, 0);
      const bool page_ok = !((t.bad >> u) & 1u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = page_ok && (tb + 16 * u + 4 * G + r < lim);
        s[u][r] = valid ? sc[r] * qs : neg_inf();
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
    if (__ballot(live && mn > m)) {
      // Some row's running max moved: rescale l and that row's accumulators.
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
    // P as the sum of two bf16 tiles, hi = bf16(p) and lo = bf16(p - hi):
    // the product then carries P to about 2^-17 relative instead of the
    // 2^-9 of one bf16 rounding, which matters when a row sees few keys.
    bf16x8 phi, plo;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 h = (__bf16)p[u][r];
        phi[4 * u + r] = h;
        plo[4 * u + r] = (__bf16)(p[u][r] - (float)h);
      }
    // B operand of MFMA j: element e = V[key of slot e][dim 8c + j].
    if constexpr (kFp8) {
      // Interleave the bytes of the two keys of each slot pair first (one
      // v_perm_b32 per 2 dims), so that each conversion yields a finished
      // operand word: 6 instructions per key pair and 4 dims instead of 8.
      u32x4 w[8];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t x0 = t.v[2 * q2][h], x1 = t.v[2 * q2 + 1][h];   // dims 4h .. 4h+3 of the two keys
          const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
          const uint32_t hi = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
          w[4 * h][q2] = e4m3x2_bf16x2<false>(lo);
          w[4 * h + 1][q2] = e4m3x2_bf16x2<true>(lo);
          w[4 * h + 2][q2] = e4m3x2_bf16x2<false>(hi);
          w[4 * h + 3][q2] = e4m3x2_bf16x2<true>(hi);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, __builtin_bit_cast(bf16x8, w[j]), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, __builtin_bit_cast(bf16x8, w[j]), acc[j], 0, 0, 0);
      }
    } else {
      // t.v[e]: dims 8c .. 8c+7 of key slot e as four bf16 pairs.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 w;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t x0 = t.v[2 * q2][j >> 1];
          const uint32_t x1 = t.v[2 * q2 + 1][j >> 1];
          w[q2] = (j & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        }
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, __builtin_bit_cast(bf16x8, w), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, __builtin_bit_cast(bf16x8, w), acc[j], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void to_lds(float* sm_m, float* sm_l, float* sm_acc, int wave) {
    const float lt = across_sum<16>(l);   // row c's denominator over the wave
    if (G == 0 && c < rows) {
      sm_m[wave * kMaxRows + c] = m;
      sm_l[wave * kMaxRows + c] = lt;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * G + r;
      if (h < rows) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm_acc[(wave * kMaxRows + h) * D + 8 * c + j] = acc[j][r];
      }
    }
  }

  // Balanced mode: this wave's piece of a segment (all its rows) is a record.
  template <bool kCoherent>
  __device__ __forceinline__ void to_record(const PartialLaunch& a, int slot) {
    const float lt = across_sum<16>(l);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * G + r;
      const float lh = __shfl(lt, h);
      const float mh = __shfl(m, h);
      if (h < rows) {
        const float inv = mh == neg_inf() ? 0.0f : vs / lh;
        float* rec = a.o_part + (int64_t)slot * rows * D;
        const int off = (h * D + 8 * c) * 4;
        put4(rec, off, f32x4{acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv}, kCoherent);
        put4(rec, off + 16, f32x4{acc[4][r] * inv, acc[5][r] * inv, acc[6][r] * inv, acc[7][r] * inv}, kCoherent);
      }
    }
    if (G == 0 && c < rows) put1(a.lse_part + (int64_t)slot * rows + c, record_lse(m, lt), kCoherent);
  }

  // Single launch, a piece that is its whole segment: write the final rows
  // c0.. of KV head kvh in b directly.
  __device__ __forceinline__ void to_output(const PartialLaunch& a, int b, int kvh, int c0) {
    const float lt = across_sum<16>(l);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * G + r;
      const float lh = __shfl(lt, h);
      const float mh = __shfl(m, h);
      if (h < rows) {
        const float inv = mh == neg_inf() ? 0.0f : vs / lh;
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = acc[j][r] * inv;
        store_out_vec<8>(a, out_row(a, b, kvh, c0 + h) * D + 8 * c, o);
      }
    }
    if (a.lse_out && G == 0 && c < rows) a.lse_out[out_row(a, b, kvh, c0 + c)] = record_lse(m, lt);
  }
};

// ---------------------------------------------------------------------------
// Single-launch merge (fd_decode). Records are written with agent-coherent
// stores; once a wave's (or workgroup's) records are complete -- s_waitcnt
// vmcnt(0) -- it counts them on their segment's counter with a relaxed
// agent-scope atomic (device atomics are coherent across XCDs). The caller
// that completes a segment's count reads its records with agent-coherent
// loads, merges them, and puts the counter back to zero. The counting
// happens after the K/V stream, so no wait drains the loads in flight.
//
// Why no cache-wide writeback or invalidate is needed: in the gfx942-family
// memory model (gfx950 included), an agent-scope release is an L2 writeback
// (buffer_wbl2 sc1) followed by a wait for every earlier store, and an
// agent-scope acquire is an L2 invalidate (buffer_inv sc1); the writeback and
// the invalidate exist for stores and loads WITHOUT the sc1 policy, while an
// sc1 access -- the encoding of a relaxed agent-scope atomic load or store --
// is coherent across the agent by itself. Every record word here is written
// by an sc1 store and read by sc1 loads, so what remains of the release is the
// wait before the counting atomic (stores_done), and of the acquire that the
// record loads are issued only after the count is known (counted). The
// language-level fences measured 2-3x slower (a writeback per worker).
// ---------------------------------------------------------------------------
// Wait until this wave's earlier stores are complete; the compiler may not
// move memory operations across it.
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt, expcnt and lgkmcnt all 0
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Merging in the single launch. A lane takes 8 consecutive dims of one row
// (D/8 lanes a row, 512/D rows a wave) and sweeps its records once, keeping a
// running maximum and rescaling its sums when it moves -- the online form of
// the combine kernel's sums -- with kUnroll records' loads in flight at a
// time (8; 16 in the MFMA kernels' split-mode tail, which has the registers).
// Records are read with 16-byte buffer loads carrying the agent-coherent cache
// policy. Row r's record s sits at byte o_off + s * o_rec of the buffer at
// o_base (its LSE at l_off + s * l_rec of l_base); both bases are wave-uniform.
struct MergeAcc {
  float m, wsum, acc[8];
  __device__ __forceinline__ void clear() {
    m = neg_inf();
    wsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  }
  // Fold in a record (ls = its LSE) or another partial sum with maximum ls:
  // both bring the two sides to the larger maximum.
  __device__ __forceinline__ void add(float ls, float ws, const float* x) {
    if (ls == neg_inf()) return;
    const float mn = fmaxf(m, ls);
    const float keep = m == neg_inf() ? 0.0f : expf(m - mn);
    const float w = expf(ls - mn);
    wsum = wsum * keep + ws * w;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e] * keep);
    m = mn;
  }
};

// Sweeps this lane's records s_first, s_first + s_step, ... (< count): the
// loop runs n_max rounds for every lane of the wave (n_max covers the lane
// with the most records) so that the loads stay outside divergent branches
// and a batch's loads are all in flight together; a lane past its last
// record reloads record 0 and gives it no weight.
template <int kUnroll = 8, int kPolicy = kCoherentPolicy>
__device__ __forceinline__ void merge_sweep(MergeAcc& st, const float* o_base, int o_off, int o_rec,
                                            const float* l_base, int l_off, int l_rec, int s_first, int s_step,
                                            int count, int n_max) {
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(o_base, kWholeRange);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(l_base, kWholeRange);
  for (int i0 = 0; i0 < n_max; i0 += kUnroll) {
    float ls[kUnroll];
    u32x4 x0[kUnroll], x1[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int s = s_first + (i0 + k) * s_step;
      const bool ok = s < count;
      const int sc = ok ? s : 0;
      const float l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, l_off + sc * l_rec, 0,
                                                                                     kPolicy));
      x0[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, o_off + sc * o_rec, 0,
                                                                              kPolicy));
      x1[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, o_off + sc * o_rec + 16, 0,
                                                                              kPolicy));
      ls[k] = ok ? l : neg_inf();
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = as_f32(x0[k][e]);
        x[4 + e] = as_f32(x1[k][e]);
      }
      st.add(ls[k], 1.0f, x);
    }
  }
}

// Write a merged row's 8 dims d0.. with one 16-byte (bf16) or two 16-byte
// (fp32) stores: out = acc / wsum, lse = m + log(wsum); a row whose records
// were all empty gets 0 and -inf.
template <class Launch>
__device__ __forceinline__ void store_row(const Launch& a, const MergeAcc& st, int64_t row, int d0, int D) {
  const bool any = st.m != neg_inf();
  const float inv = any ? 1.0f / st.wsum : 0.0f;
  const int64_t idx = row * D + d0;
  if (a.out_dtype == FD_BF16) {
    u32x4 packed;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      packed[q] = (uint32_t)to_bf16_rne(st.acc[2 * q] * inv) | ((uint32_t)to_bf16_rne(st.acc[2 * q + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + idx) = packed;
  } else {
    float* o = reinterpret_cast<float*>(a.out) + idx;
    *reinterpret_cast<f32x4*>(o) = f32x4{st.acc[0] * inv, st.acc[1] * inv, st.acc[2] * inv, st.acc[3] * inv};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{st.acc[4] * inv, st.acc[5] * inv, st.acc[6] * inv, st.acc[7] * inv};
  }
  if (a.lse_out && d0 == 0) a.lse_out[row] = any ? st.m + logf(st.wsum) : neg_inf();
}

// Lane roles in a merge pass over rows rp .. rp + 512/D - 1 of R: with fewer
// rows than a wave holds, the rows' lanes repeat `groups` times, each copy
// taking every groups-th record, and group 0 collects the others.
struct PassLanes {
  int r;        // row of this lane
  int rows;     // rows in this pass
  int group;    // which copy of the rows
  int groups;   // copies
  bool live;    // the lane holds a row of the pass
};
template <int D>
__device__ __forceinline__ PassLanes pass_lanes(int R, int rp) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kPass = 64 / kLanesPerRow;
  const int q = lane_id() / kLanesPerRow;
  PassLanes p;
  p.rows = min(kPass, R - rp);
  p.groups = kPass / p.rows;
  p.group = q / p.rows;
  p.live = p.group < p.groups;
  p.r = rp + (p.live ? q - p.group * p.rows : 0);
  return p;
}
// Group 0's lanes add the partial sums of the other copies of their row
// (read from a copy taken before any lane adds anything).
template <int D>
__device__ __forceinline__ void gather_groups(MergeAcc& st, const PassLanes& p) {
  constexpr int kLanesPerRow = D / 8;
  const MergeAcc own = st;
  for (int k = 1; k < p.groups; ++k) {
    const int src = lane_id() + k * p.rows * kLanesPerRow;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __shfl(own.acc[e], src);
    const float m = __shfl(own.m, src);
    const float ws = __shfl(own.wsum, src);
    st.add(m, ws, x);
  }
}

// Count one finished record of segment `seg` (one lane calls it). True for
// the caller that completes the segment's `total`.
__device__ __forceinline__ bool count_piece(const PartialLaunch& a, int64_t seg, int total) {
  const int old = __hip_atomic_fetch_add(a.counters + seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old == total - 1;
}

// Between the count that found a segment complete and the loads of its
// records: the compiler may not move those loads above the count.
__device__ __forceinline__ void counted() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void reset_count(const PartialLaunch& a, int64_t seg) {
  __hip_atomic_store(a.counters + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Split driver: the chunk [split * C, min((split + 1) * C, L_b)) of one
// (sequence, segment), four waves taking its tiles in turn.
// ---------------------------------------------------------------------------
template <class E, bool kPaged, int kEsz>
__device__ __forceinline__ void run_split(const PartialLaunch& a, E& e, float* sm_m, float* sm_l, float* sm_acc,
                                          float (*sm_part)[64][10], int stride_h) {
  constexpr int kTile = E::kTile;
  const int R = a.geo.rows_per_seg;
  const int tiles_h = a.geo.segs_per_seq / a.num_kv_heads;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y / tiles_h;
  const int c0 = (blockIdx.y - kvh * tiles_h) * R;
  const int b = blockIdx.z;
  const int wave = wave_id();
  const int len = clamp_len(a, b);
  const int lo = split * a.geo.chunk_len;
  const int hi = min(lo + a.geo.chunk_len, len);

  // Tiles of this wave: lo + (wave + n * kWaves) * kTile. The query rows
  // and the first tile are requested together. The next tile is always
  // loaded before the current one is used (past hi its descriptors are
  // empty and the loads fetch nothing), so loads stay in flight across the
  // math.
  constexpr int kStep = kWaves * kTile;
  int tb = lo + wave * kTile;
  const bool has_tiles = tb < hi;
  typename E::Source src;
  src.init(a, b, kvh, hi, kEsz);
  typename E::Tile t0, t1;
  t0.buf = 0;
  t1.buf = 1;
  e.fetch_q(a, b, kvh, c0);
  if (has_tiles) e.load(t0, src, tb);
  e.window(a, kvh, c0, hi, len);
  e.reset();
  if (has_tiles) {
    for (;;) {
      e.load(t1, src, tb + kStep);
      e.compute(t0, tb);
      tb += kStep;
      if (tb >= hi) break;
      e.load(t0, src, tb + kStep);
      e.compute(t1, tb);
      tb += kStep;
      if (tb >= hi) break;
    }
  }
  if constexpr (E::kStageBytes > 0)
    __syncthreads();   // every wave is past its tiles: the merge area reuses the K stages
  e.to_lds(sm_m, sm_l, sm_acc, wave);
  __syncthreads();
  merge_waves<E::kD>(a, sm_m, sm_l, sm_acc, R, stride_h, b, kvh, c0, split, e.vs);
  if (a.out == nullptr) return;

  // Single launch: the workgroup that writes the last of the segment's
  // num_splits records merges them.
  __shared__ int last;
  stores_done();     // this wave's record stores are complete ...
  __syncthreads();   // ... and so are every other wave's
  const int64_t seg = (int64_t)b * a.geo.segs_per_seq + blockIdx.y;
  if (threadIdx.x == 0) last = count_piece(a, seg, a.geo.num_splits);
  __syncthreads();
  if (!last) return;
  counted();
  // Per pass of 512 / D rows, the four waves sweep every fourth record and
  // wave 0 adds their partial sums.
  const int S = a.geo.num_splits;
  constexpr int kD = E::kD;
  constexpr int kLanesPerRow = kD / 8;
  constexpr int kPass = 64 / kLanesPerRow;
  const int lane = lane_id();
  const int d0 = 8 * (lane % kLanesPerRow);
  for (int rp = 0; rp < R; rp += kPass) {
    const PassLanes pl = pass_lanes<kD>(R, rp);
    const int64_t row0 = out_row(a, b, kvh, c0 + rp);
    const int64_t drow = out_row(a, b, kvh, c0 + pl.r) - row0;
    MergeAcc st;
    st.clear();
    merge_sweep<E::kTailUnroll>(st, a.o_part + row0 * S * kD, (int)((drow * S * kD + d0) * 4), kD * 4, a.lse_part + row0 * S,
                (int)(drow * S * 4), 4, pl.live ? wave + kWaves * pl.group : S, kWaves * pl.groups, S,
                (S - wave + kWaves * pl.groups - 1) / (kWaves * pl.groups));
    gather_groups<kD>(st, pl);
    float* mine = sm_part[wave][lane];
    mine[0] = st.m;
    mine[1] = st.wsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) mine[2 + e] = st.acc[e];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < kWaves; ++w) st.add(sm_part[w][lane][0], sm_part[w][lane][1], &sm_part[w][lane][2]);
      if (pl.live && pl.group == 0) store_row(a, st, out_row(a, b, kvh, c0 + pl.r), d0, kD);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) reset_count(a, seg);
}

// ---------------------------------------------------------------------------
// Balanced driver. Sequence b has T_b = ceil(L_b / kTile) tiles per segment
// and J segments (KV heads x row tiles); segments are laid end to end in
// (b, segment) order, so T = J * sum_b T_b tiles in all. Worker p takes a
// consecutive run of them (Partition: ceil(T / workers) each unless the
// plan gives leading workers a larger share) and streams it; tile t of a
// segment starting at tile offset o sits at o + t.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// The balanced partition of the T tiles over the workers: the first w1
// workers take q1 tiles each, the others q2 (q1 = q2 and w1 = 0 unless the
// plan gives leading workers a larger share), the last ones possibly fewer
// or none. The partial kernel, the combine and the single-launch merge all
// derive it from the same Geometry and T.
// The host keeps the batch's tile count below 2^31, so tile offsets, shares
// and worker indices fit 32 bits and the divisions run in 32 bits (a 64-bit
// division is a long instruction sequence on the way to the first loads);
// only the leading-share product 100 T needs 64 bits.
struct Partition {
  int64_t q1, q2, w1;
  __device__ __forceinline__ int64_t first(int64_t w) const { return w < w1 ? w * q1 : w1 * q1 + (w - w1) * q2; }
  __device__ __forceinline__ int64_t size(int64_t w) const { return w < w1 ? q1 : q2; }
  __device__ __forceinline__ int64_t owner(int64_t x) const {
    const int64_t lead = w1 * q1;
    return x < lead ? (int64_t)((uint32_t)x / (uint32_t)q1)
                    : w1 + (int64_t)((uint32_t)(x - lead) / (uint32_t)q2);
  }
};
__device__ __forceinline__ Partition partition(const Geometry& g, int64_t T) {
  Partition p;
  const int64_t W = g.workers;
  if (g.lead_pct <= 0) {
    p.w1 = 0;
    p.q1 = p.q2 = max(1u, ((uint32_t)T + (uint32_t)W - 1u) / (uint32_t)W);
    return p;
  }
  const int64_t pct = g.lead_pct;
  p.w1 = min((int64_t)g.lead_workers, W);
  p.q2 = max((int64_t)1, (100 * T + p.w1 * pct + (W - p.w1) * 100 - 1) / (p.w1 * pct + (W - p.w1) * 100));
  p.q1 = max((int64_t)1, (p.q2 * pct + 99) / 100);
  return p;
}

struct Cursor {
  int b;      // sequence
  int j;      // segment within the sequence
  int t;      // key tile within the segment
  int tiles;  // T_b
  int len;    // L_b (clamped)
  int pre;    // sum of T_b' over b' < b
  int64_t v;  // offset of tile t in the partition's tile order
};

// kFused: the single-launch variant (fd_decode), which also merges.
template <class E, bool kPaged, int kEsz, bool kFused>
__device__ __forceinline__ void run_balanced(const PartialLaunch& a, E& e) {
  constexpr int kTile = E::kTile;
  const int worker = blockIdx.x * kWaves + wave_id();
  if (worker >= a.geo.workers) return;
  const int lane = lane_id();
  const int B = a.batch;
  const int J = a.geo.segs_per_seq;
  const int R = a.geo.rows_per_seg;
  const int tiles_h = J / a.num_kv_heads;
  const int rows_per_seq = a.geo.q_len * a.num_q_heads;
  // The batch's lengths, 64 sequences a round: lane l of round r holds
  // sequence 64 r + l. The first kCachedRounds rounds are loaded at once, all
  // loads in flight together, and kept in registers for both passes below and
  // for the cursor's moves from one sequence to the next (which then wait for
  // no load before the next tile's loads can go out); later rounds of a larger
  // batch are read where they are needed.
  // (Four named values rather than an array: an array indexed by a runtime
  // round would be moved out of registers.)
  constexpr int kCachedRounds = 4;
  const int len0 = clamp_len(a, min(lane, B - 1));
  const int len1 = clamp_len(a, min(64 + lane, B - 1));
  const int len2 = clamp_len(a, min(128 + lane, B - 1));
  const int len3 = clamp_len(a, min(192 + lane, B - 1));
  auto cached = [&](int r) { return r == 0 ? len0 : r == 1 ? len1 : r == 2 ? len2 : len3; };
  auto round_len = [&](int r) {   // this lane's sequence of round r (r wave-uniform)
    return r < kCachedRounds ? cached(r) : clamp_len(a, min(64 * r + lane, B - 1));
  };
  auto seq_len = [&](int b) {     // sequence b's length (b wave-uniform)
    return b < 64 * kCachedRounds ? __builtin_amdgcn_readlane(cached(b >> 6), b & 63) : clamp_len(a, b);
  };

  // Pass 1: T. Worker 0 also publishes the running tile counts for the combine.
  int run = 0;
  for (int cb = 0, r = 0; cb < B; cb += 64, ++r) {
    const int bl = cb + lane;
    const int tl = bl < B ? (round_len(r) + kTile - 1) / kTile : 0;
    const int incl = wave_incl_scan(tl);
    if (worker == 0 && bl < B) {
      a.tile_prefix[bl] = run + incl - tl;
      // Single launch: a sequence with no key has no piece to merge; its rows
      // are written here as 0 and -inf.
      if (kFused && tl == 0) {
        for (int h = 0; h < rows_per_seq; ++h) {
          const int64_t row = (int64_t)bl * rows_per_seq + h;
          for (int d = 0; d < E::kD; ++d) store_out(a, row * E::kD + d, 0.0f);
          if (a.lse_out) a.lse_out[row] = neg_inf();
        }
      }
    }
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  if (worker == 0 && lane == 0) a.tile_prefix[B] = run;
  const int64_t T = (int64_t)J * run;
  const Partition part = partition(a.geo, T);
  const int64_t x0 = part.first(worker);
  if (x0 >= T) return;
  const int64_t x1 = min(x0 + part.size(worker), T);   // the run is tiles [x0, x1)

  // Pass 2: the cursor at tile x: sequence b holds it when b is the last
  // sequence with J * prefix_b <= x. (The single launch calls this again
  // after its run instead of keeping the run's start cursor live through the
  // stream.)
  auto locate = [&](int64_t x) {
    int best_b = 0, best_pre = 0, pre = 0;
    for (int cb = 0, r = 0; cb < B; cb += 64, ++r) {
      const int bl = cb + lane;
      const int tl = bl < B ? (round_len(r) + kTile - 1) / kTile : 0;
      const int incl = wave_incl_scan(tl);
      const int excl = pre + incl - tl;
      const uint64_t ok = __ballot(bl < B && (int64_t)J * excl <= x);
      const int cnt = __popcll(ok);
      if (cnt > 0) {
        best_b = cb + cnt - 1;
        best_pre = __builtin_amdgcn_readlane(excl, cnt - 1);
      }
      if (cnt < 64) break;
      pre += __builtin_amdgcn_readlane(incl, 63);
    }
    Cursor c;
    c.b = best_b;
    c.pre = best_pre;
    c.len = seq_len(best_b);
    c.tiles = (c.len + kTile - 1) / kTile;
    const int rem = (int)(x - (int64_t)J * best_pre);
    c.j = rem / c.tiles;
    c.t = rem - c.j * c.tiles;
    c.v = x;
    return c;
  };
  Cursor cur = locate(x0);
  auto advance = [&](Cursor x) {
    ++x.v;
    if (++x.t == x.tiles) {
      x.t = 0;
      if (++x.j == J) {
        x.j = 0;
        // Only called while tiles remain, so a later sequence has tiles; the
        // bound keeps every length read inside seq_lens regardless.
        while (x.b + 1 < B) {
          x.pre += x.tiles;
          ++x.b;
          x.len = seq_len(x.b);
          x.tiles = (x.len + kTile - 1) / kTile;
          if (x.tiles > 0) break;
        }
      }
    }
    return x;
  };
  auto kv_head = [&](const Cursor& x) { return x.j / tiles_h; };
  auto first_row = [&](const Cursor& x) { return (x.j - (x.j / tiles_h) * tiles_h) * R; };

  // Single launch: merge segment (b, j), whose records are slots
  // seg + p0 .. seg + p0 + total - 1, once every piece of it is counted.
  auto merge_segment = [&](int b, int j, int seg, int64_t p0, int total) {
    const int kvh = j / tiles_h, c0 = (j - kvh * tiles_h) * R;
    const int64_t slot = seg + p0;
    constexpr int kD = E::kD;
    constexpr int kLanesPerRow = kD / 8;
    constexpr int kPass = 64 / kLanesPerRow;
    const int d0 = 8 * (lane % kLanesPerRow);
    const float* ob = a.o_part + slot * R * kD;
    const float* lb = a.lse_part + slot * R;
    for (int rp = 0; rp < R; rp += kPass) {
      const PassLanes pl = pass_lanes<kD>(R, rp);
      MergeAcc st;
      st.clear();
      merge_sweep(st, ob, (pl.r * kD + d0) * 4, R * kD * 4, lb, pl.r * 4, R * 4, pl.live ? pl.group : total,
                  pl.groups, total, (total + pl.groups - 1) / pl.groups);
      gather_groups<kD>(st, pl);
      if (pl.live && pl.group == 0) store_row(a, st, out_row(a, b, kvh, c0 + pl.r), d0, kD);
    }
    if (lane == 0) reset_count(a, seg);
  };
  typename E::Source sc, sn;
  sc.init(a, cur.b, kv_head(cur), cur.len, kEsz);
  typename E::Tile t0, t1;
  t0.buf = 0;
  t1.buf = 1;
  // Load order. By default a step requests tile i+1 and then computes tile
  // i. With kAhead (the kernels that stage K through LDS) tile i+1 is
  // already in flight when tile i is computed, and tile i+2 is requested into
  // tile i's buffer right after, before a record that tile i closes is
  // written. Measured on MI355X (same box, two A/B rounds): the fp8 paged
  // batch 1.5 % faster that way, the register-K kernels 0.2 % faster to 2 %
  // slower (more registers live across the loop), so only the LDS-K
  // kernels take it.
  constexpr bool kAhead = E::kStageBytes > 0;
  bool nx_in_run = cur.v + 1 < x1;   // kAhead: nxa, the tile after cur, is in the run
  Cursor nxa = cur;
  e.fetch_q(a, cur.b, kv_head(cur), first_row(cur));
  e.load(t0, sc, cur.t * kTile);
  if constexpr (kAhead) {
    sn = sc;
    if (nx_in_run) {
      nxa = advance(cur);
      if (nxa.b != cur.b || nxa.j != cur.j) sn.init(a, nxa.b, kv_head(nxa), nxa.len, kEsz);
    } else {
      sn.none();
    }
    e.load(t1, sn, nxa.t * kTile);
  }
  e.window(a, kv_head(cur), first_row(cur), cur.len, cur.len);
  e.reset();

  // Closing the piece that tile cur ends (fresh: the next tile, n, opens
  // another). In the single launch a piece that is its whole segment -- it
  // starts at the segment's first tile (every piece but the run's first does)
  // and ends at its last -- is written straight to the output and never
  // counted.
  bool from_first = cur.t == 0;   // the open piece starts at its segment's first tile
  auto close_piece = [&](bool fresh, const Cursor& n) {
    if (kFused && from_first && cur.t == cur.tiles - 1)
      e.to_output(a, cur.b, kv_head(cur), first_row(cur));
    else
      e.template to_record<kFused>(a, cur.b * J + cur.j + worker);
    from_first = true;   // every later piece opens its segment
    e.reset();
    if (fresh) e.window(a, kv_head(n), first_row(n), n.len, n.len);
  };

  // kAhead step: compute tile cur (in `now`; nxa is in flight in the other
  // buffer), request the next piece's query rows if nxa opens one (q is dead
  // now; before the tile load, so that waiting for them leaves that load in
  // flight), request the tile after nxa (or nothing) into `now`, then close
  // the piece if cur ends it.
  auto step_ahead = [&](typename E::Tile& now) -> bool {
    e.compute(now, cur.t * kTile);
    const bool fresh = nx_in_run && (nxa.b != cur.b || nxa.j != cur.j);
    if (fresh) e.fetch_q(a, nxa.b, kv_head(nxa), first_row(nxa));
    const bool more2 = nx_in_run && nxa.v + 1 < x1;
    Cursor n2 = nxa;
    typename E::Source s2 = sn;
    if (more2) {
      n2 = advance(nxa);
      if (n2.b != nxa.b || n2.j != nxa.j) s2.init(a, n2.b, kv_head(n2), n2.len, kEsz);
    } else {
      s2.none();
    }
    e.load(now, s2, n2.t * kTile);
    if (!nx_in_run || fresh) close_piece(fresh, nxa);
    const bool go_on = nx_in_run;
    cur = nxa;
    nxa = n2;
    sn = s2;
    nx_in_run = more2;
    return go_on;
  };

  // Default step: prefetch tile i+1 (or nothing), update with tile i, and
  // close the record when tile i ends a segment piece; the next piece's query
  // rows are loaded once tile i is computed (q is dead then).
  auto step = [&](typename E::Tile& now, typename E::Tile& later) -> bool {
    const bool more = cur.v + 1 < x1;
    Cursor nx = cur;
    bool fresh = false;
    sn = sc;
    if (more) {
      nx = advance(cur);
      fresh = nx.b != cur.b || nx.j != cur.j;
      if (fresh) sn.init(a, nx.b, kv_head(nx), nx.len, kEsz);
    } else {
      sn.none();
    }
    e.load(later, sn, nx.t * kTile);
    e.compute(now, cur.t * kTile);
    if (!more || fresh) {
      if (fresh) e.fetch_q(a, nx.b, kv_head(nx), first_row(nx));
      close_piece(fresh, nx);
    }
    cur = nx;
    sc = sn;
    return more;
  };
  if constexpr (kAhead) {
    for (;;) {
      if (!step_ahead(t0)) break;
      if (!step_ahead(t1)) break;
    }
  } else {
    for (;;) {
      if (!step(t0, t1)) break;
      if (!step(t1, t0)) break;
    }
  }
  if constexpr (kFused) {
    // Count this worker's pieces -- one per segment its run touched, in
    // order -- now that its records are complete: lane i counts piece i
    // (up to 64 at a time, all atomics in one instruction); the pieces that
    // complete their segment are then merged one after another. A segment
    // of one piece (total 1) was written out above and has no count.
    stores_done();
    Cursor x = locate(x0);
    bool more = true;
    while (more) {
      int my_seg = 0, my_b = 0, my_j = 0, my_total = 0;
      int64_t my_p0 = 0;
      int k = 0;
      for (; k < 64 && more; ++k) {
        const int64_t key0 = (int64_t)J * x.pre + (int64_t)x.j * x.tiles;   // the segment's first tile
        const int64_t p0 = part.owner(key0), p1 = part.owner(key0 + x.tiles - 1);
        if (lane == k) {
          my_seg = x.b * J + x.j;
          my_b = x.b;
          my_j = x.j;
          my_p0 = p0;
          my_total = (int)(p1 - p0 + 1);
        }
        x.v += x.tiles - 1 - x.t;   // the segment's last key tile
        x.t = x.tiles - 1;
        if (x.v + 1 >= x1)
          more = false;
        else
          x = advance(x);
      }
      const bool last = lane < k && my_total > 1 && count_piece(a, my_seg, my_total);
      const uint64_t completed = __ballot(last);
      counted();
      for (uint64_t lasts = completed; lasts; lasts &= lasts - 1) {
        const int i = __builtin_ctzll(lasts);
        merge_segment(__builtin_amdgcn_readlane(my_b, i), __builtin_amdgcn_readlane(my_j, i),
                      __builtin_amdgcn_readlane(my_seg, i),
                      ((int64_t)__builtin_amdgcn_readlane((int)(my_p0 >> 32), i) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)my_p0, i),
                      __builtin_amdgcn_readlane(my_total, i));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------
template <typename KV, int D, int GT, bool kPaged, int kMode>
__global__ __launch_bounds__(kThreads) void partial_valu(PartialLaunch a) {
  using E = ValuEngine<KV, D, GT, kPaged>;
  E e;
  e.init(a, lane_id());
  if constexpr (kMode == FD_MODE_SPLITS) {
    __shared__ float sm_m[kWaves * GT];
    __shared__ float sm_l[kWaves * GT];
    __shared__ float sm_acc[kWaves * GT * D];
    __shared__ float sm_part[kWaves][64][10];
    run_split<E, kPaged, sizeof(KV)>(a, e, sm_m, sm_l, sm_acc, sm_part, GT);
  } else {
    run_balanced<E, kPaged, sizeof(KV), kMode == kModeBalancedFused>(a, e);
  }
}

// LDS of the MFMA kernel: the K stages (fp8), and in split mode the four
// waves' merge area, which reuses the K stages once every wave is past its
// tiles.
template <class E, bool kSplit>
struct MfmaLds {
  static constexpr int kMergeBytes = 4 * (2 * kWaves * E::kMaxRows + kWaves * E::kMaxRows * E::D + kWaves * 64 * 10);
  static constexpr int kStage = kWaves * E::kStageBytes;
  static constexpr int kPool = !kSplit ? (kStage > 16 ? kStage : 16) : (kStage > kMergeBytes ? kStage : kMergeBytes);
};

template <bool kPaged, bool kFp8, int kMode>
__global__ __launch_bounds__(kThreads, 2) void partial_mfma_d128(PartialLaunch a) {
  using E = MfmaEngine<kPaged, kFp8>;
  using L = MfmaLds<E, kMode == FD_MODE_SPLITS>;
  __shared__ __attribute__((aligned(16))) char pool[L::kPool];
  E e;
  e.init(a, lane_id());
  e.kst = (lds_char*)(pool + wave_id() * E::kStageBytes);
  if constexpr (kMode == FD_MODE_SPLITS) {
    float* sm_m = reinterpret_cast<float*>(pool);
    float* sm_l = sm_m + kWaves * E::kMaxRows;
    float* sm_acc = sm_l + kWaves * E::kMaxRows;
    auto sm_part = reinterpret_cast<float (*)[64][10]>(sm_acc + kWaves * E::kMaxRows * E::D);
    run_split<E, kPaged, E::kEsz>(a, e, sm_m, sm_l, sm_acc, sm_part, E::kMaxRows);
  } else {
    run_balanced<E, kPaged, E::kEsz, kMode == kModeBalancedFused>(a, e);
  }
}

// ---------------------------------------------------------------------------
// Combine, row by row. Per output row: M = max_s LSE_s over the row's records; w_s =
// exp(LSE_s - M), zero for an empty one (LSE = -inf); out = sum_s w_s o_s /
// sum_s w_s; lse_out = M + log(sum_s w_s). A row with no valid key gets 0 and
// -inf.
//
// kWpr waves serve one row. A lane holds 8 consecutive dims (two 16-byte
// loads per record), so D/8 lanes cover a record and the wave's 64/(D/8)
// lane groups, across kWpr waves, take the records in turn. Each group merges
// its records in one pass with a running maximum ([INFRA] 2.6, the online
// form of the same sums), eight records' loads in flight at once; the groups
// (shuffles) and waves (LDS) are then brought to the row's maximum and added.
// ---------------------------------------------------------------------------
template <typename OutT, int D, int kWpr>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineLaunch a) {
  constexpr int kLanesPerRec = D / 8;
  constexpr int kGroupsPerWave = 64 / kLanesPerRec;
  constexpr int kGroups = kGroupsPerWave * kWpr;
  constexpr int kRowsPerBlock = kWaves / kWpr;
  __shared__ float sm[kWaves][kLanesPerRec][9];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int rows = a.batch * a.geo.q_len * a.num_q_heads;
  const int row = blockIdx.x * kRowsPerBlock + wave / kWpr;
  const int wr = wave % kWpr;                       // wave within the row
  const int grp = wr * kGroupsPerWave + lane / kLanesPerRec;
  const int sl = lane % kLanesPerRec;               // dims 8*sl .. 8*sl+7
  const bool live_row = row < rows;
  const int r = live_row ? row : 0;

  // The row's records: `count` of them, `ostride` floats apart in o_part and
  // `lstride` apart in lse_part.
  int64_t obase, lbase, ostride, lstride;
  int count;
  if (a.geo.mode == FD_MODE_SPLITS) {
    count = a.geo.num_splits;
    obase = (int64_t)r * count * D;
    lbase = (int64_t)r * count;
    ostride = D;
    lstride = 1;
  } else {
    // Output row r = (b, t, h) is row c = t * g + (h - kvh * g) of KV head
    // kvh's rows, held by segment kvh * tiles_h + c / R as its row c % R.
    // The row is wave-uniform, so this is scalar work: the tile counts come
    // in as scalar loads, and every quantity fits 32 bits (the host keeps
    // the batch's tile count below 2^31).
    const int g = a.num_q_heads / a.num_kv_heads;
    const int hps = a.geo.rows_per_seg;
    const int J = a.geo.segs_per_seq;
    const int tiles_h = J / a.num_kv_heads;
    const int rows_per_seq = a.geo.q_len * a.num_q_heads;
    const int b = r / rows_per_seq;
    const int i = r - b * rows_per_seq;
    const int t = i / a.num_q_heads;
    const int h = i - t * a.num_q_heads;
    const int kvh = h / g;
    const int cr = t * g + (h - kvh * g);
    const int ti = cr / hps;
    const int hs = cr - ti * hps;
    const int j = kvh * tiles_h + ti;
    const int pre = load_uniform(a.tile_prefix, b);
    const int tb = load_uniform(a.tile_prefix, b + 1) - pre;
    const int T = J * load_uniform(a.tile_prefix, a.batch);
    const Partition part = partition(a.geo, T);
    // tb = the sequence's tiles per segment (0 if it has no key). The
    // range is clamped to the workers' slots, so that no workspace contents
    // can send a read outside the records.
    const int key0 = J * pre + j * tb;
    const int W = a.geo.workers;
    const int p0 = tb > 0 ? min(max((int)part.owner(key0), 0), W - 1) : 0;
    const int p1 = tb > 0 ? min(max((int)part.owner(key0 + tb - 1), p0 - 1), W - 1) : -1;
    count = p1 - p0 + 1;
    const int64_t slot = (int64_t)b * J + j + p0;
    obase = (slot * hps + hs) * D;
    lbase = slot * hps + hs;
    ostride = (int64_t)hps * D;
    lstride = hps;
  }
  const float* lse = a.lse_part + lbase;
  const float* o = a.o_part + obase + 8 * sl;

  // One pass over the records, kUnroll per lane group at a time with all of
  // their loads in flight: each group keeps a running maximum m and rescales
  // its sums when it moves (the online form of the same merge), so no
  // separate pass for the row's maximum is needed. Empty records (LSE = -inf)
  // weigh zero.
  constexpr int kUnroll = 8;
  float m = neg_inf(), wsum = 0.0f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  if (live_row) {
    for (int s0 = grp; s0 < count; s0 += kGroups * kUnroll) {
      float ls[kUnroll];
      f32x4 x0[kUnroll], x1[kUnroll];
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        const int s = s0 + k * kGroups;
        const bool ok = s < count;
        const int sc = ok ? s : 0;
        ls[k] = ok ? lse[sc * lstride] : neg_inf();
        x0[k] = *reinterpret_cast<const f32x4*>(o + sc * ostride);
        x1[k] = *reinterpret_cast<const f32x4*>(o + sc * ostride + 4);
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
        if (ls[k] == neg_inf()) continue;
        const float mn = fmaxf(m, ls[k]);
        const float keep = m == neg_inf() ? 0.0f : expf(m - mn);
        const float w = expf(ls[k] - mn);
        wsum = wsum * keep + w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = fmaf(w, x0[k][e], acc[e] * keep);
          acc[4 + e] = fmaf(w, x1[k][e], acc[4 + e] * keep);
        }
        m = mn;
      }
    }
  }
  // Lane groups of this wave (then the row's waves) hold disjoint records of
  // the same dims: bring them to the common maximum and add them up.
  float M = across_max<kLanesPerRec>(m);
  if constexpr (kWpr > 1) {
    __shared__ float sm_m[kWaves];
    if (lane == 0) sm_m[wave] = M;
    __syncthreads();
    const int w0 = wave - wr;
#pragma unroll
    for (int w = 0; w < kWpr; ++w) M = fmaxf(M, sm_m[w0 + w]);
  }
  const bool any = M != neg_inf();
  const float f = (m == neg_inf()) ? 0.0f : expf(m - M);
  wsum *= f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = across_sum<kLanesPerRec>(acc[e] * f);
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

// ---------------------------------------------------------------------------
// Combine, balanced mode, a wave per segment (for batches of many segments
// with few records each). A segment's records are the contiguous slots
// seg + p0 .. seg + p1, each holding its R rows side by side, so a lane takes
// 8 dims of one row (512/D rows a pass; with fewer rows than that, copies of
// the rows' lanes take every groups-th record) and sweeps its records once
// with the online merge, eight records' loads in flight -- the same sums as
// combine_kernel, read as whole rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void combine_segments(CombineLaunch a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kPass = 64 / kLanesPerRow;
  const int J = a.geo.segs_per_seq;
  const int seg = blockIdx.x * kWaves + wave_id();
  if (seg >= a.batch * J) return;
  const int R = a.geo.rows_per_seg;
  const int tiles_h = J / a.num_kv_heads;
  const int b = seg / J;
  const int j = seg - b * J;
  const int kvh = j / tiles_h;
  const int c0 = (j - kvh * tiles_h) * R;
  // Scalar work: the tile counts are scalar loads and every quantity fits
  // 32 bits (the host keeps the batch's tile count below 2^31).
  const int pre = load_uniform(a.tile_prefix, b);
  const int tb = load_uniform(a.tile_prefix, b + 1) - pre;
  const int T = J * load_uniform(a.tile_prefix, a.batch);
  const Partition part = partition(a.geo, T);
  // The record range is clamped to the workers' slots (as in combine_kernel).
  const int key0 = J * pre + j * tb;
  const int W = a.geo.workers;
  const int p0 = tb > 0 ? min(max((int)part.owner(key0), 0), W - 1) : 0;
  const int count = tb > 0 ? min(max((int)part.owner(key0 + tb - 1), p0 - 1), W - 1) - p0 + 1 : 0;
  const int64_t slot = (int64_t)seg + p0;
  const float* ob = a.o_part + slot * R * D;
  const float* lb = a.lse_part + slot * R;
  const int d0 = 8 * (lane_id() % kLanesPerRow);
  for (int rp = 0; rp < R; rp += kPass) {
    const PassLanes pl = pass_lanes<D>(R, rp);
    MergeAcc st;
    st.clear();
    merge_sweep<8, 0>(st, ob, (pl.r * D + d0) * 4, R * D * 4, lb, pl.r * 4, R * 4, pl.live ? pl.group : count,
                   pl.groups, count, (count + pl.groups - 1) / pl.groups);
    gather_groups<D>(st, pl);
    if (pl.live && pl.group == 0) store_row(a, st, out_row(a, b, kvh, c0 + pl.r), d0, D);
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int kMode>
dim3 partial_grid(const PartialLaunch& a) {
  if (kMode == FD_MODE_SPLITS) return dim3(a.geo.num_splits, a.geo.segs_per_seq, a.batch);
  return dim3((a.geo.workers + kWaves - 1) / kWaves);
}

template <typename KV, int D, int GT, int kMode>
hipError_t launch_valu_typed(const PartialLaunch& a, hipStream_t stream) {
  const dim3 grid = partial_grid<kMode>(a);
  if (a.paged)
    hipLaunchKernelGGL((partial_valu<KV, D, GT, true, kMode>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((partial_valu<KV, D, GT, false, kMode>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename KV, int D, int kMode>
hipError_t launch_valu_d(const PartialLaunch& a, hipStream_t stream) {
  switch (a.geo.rows_per_seg) {
    case 4:
      if constexpr (!KvType<KV>::kFp8) return launch_valu_typed<KV, D, 4, kMode>(a, stream);
      return hipErrorInvalidValue;
    case 2: return launch_valu_typed<KV, D, 2, kMode>(a, stream);
    case 1: return launch_valu_typed<KV, D, 1, kMode>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename KV, int kMode>
hipError_t launch_valu(const PartialLaunch& a, hipStream_t stream) {
  return a.head_dim == 64 ? launch_valu_d<KV, 64, kMode>(a, stream) : launch_valu_d<KV, 128, kMode>(a, stream);
}

template <bool kFp8, int kMode>
hipError_t launch_mfma(const PartialLaunch& a, hipStream_t stream) {
  const dim3 grid = partial_grid<kMode>(a);
  if (a.paged)
    hipLaunchKernelGGL((partial_mfma_d128<true, kFp8, kMode>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((partial_mfma_d128<false, kFp8, kMode>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int kMode>
hipError_t launch_partial_mode(const PartialLaunch& a, hipStream_t stream) {
  if (a.path == FD_PATH_MFMA)
    return a.kv_dtype == FD_FP8_E4M3 ? launch_mfma<true, kMode>(a, stream) : launch_mfma<false, kMode>(a, stream);
  if (a.kv_dtype == FD_FP8_E4M3) return launch_valu<uint8_t, kMode>(a, stream);
  if (a.kv_dtype == FD_BF16) return launch_valu<uint16_t, kMode>(a, stream);
  return launch_valu<float, kMode>(a, stream);
}

// Segments from which a balanced batch is combined a segment per wave
// (MI355X: 4.5 against 6.6 us at 1024 segments of ~2 records; slower than the
// row-wise kernel at 128 segments of 9-17 records).
constexpr int kSegmentCombineMinSegs = 1024;

template <typename OutT, int D>
hipError_t launch_combine_typed(const CombineLaunch& a, hipStream_t stream) {
  // Waves per row grow with the records a row can hold, so long record lists
  // are read in parallel: one wave up to 32 records, two up to 63, then four.
  const int rows = a.batch * a.geo.q_len * a.num_q_heads;
  int expect = a.geo.num_splits;
  if (a.geo.mode == FD_MODE_BALANCED) {
    const int segs = a.batch * a.geo.segs_per_seq;
    expect = (a.geo.workers + segs - 1) / segs + 1;
  }
  const int wpr = expect >= 64 ? 4 : expect > 32 ? 2 : 1;
  const int rows_per_block = kWaves / wpr;
  dim3 grid((rows + rows_per_block - 1) / rows_per_block);
  if (wpr == 4)
    hipLaunchKernelGGL((combine_kernel<OutT, D, 4>), grid, dim3(kThreads), 0, stream, a);
  else if (wpr == 2)
    hipLaunchKernelGGL((combine_kernel<OutT, D, 2>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<OutT, D, 1>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <class K>
int occupancy_waves(K kernel) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kThreads, 0) != hipSuccess) return 0;
  return blocks * kWaves;
}

template <typename KV, int D, int GT>
int valu_waves(int paged) {
  return paged ? occupancy_waves(partial_valu<KV, D, GT, true, FD_MODE_BALANCED>)
               : occupancy_waves(partial_valu<KV, D, GT, false, FD_MODE_BALANCED>);
}

template <typename KV, int D>
int valu_waves_d(int rows, int paged) {
  switch (rows) {
    case 4:
      if constexpr (!KvType<KV>::kFp8) return valu_waves<KV, D, 4>(paged);
      return 0;
    case 2: return valu_waves<KV, D, 2>(paged);
    case 1: return valu_waves<KV, D, 1>(paged);
  }
  return 0;
}

template <typename KV>
int valu_waves_kv(int head_dim, int rows, int paged) {
  return head_dim == 64 ? valu_waves_d<KV, 64>(rows, paged) : valu_waves_d<KV, 128>(rows, paged);
}

template <typename KV>
int valu_tile(int head_dim) {
  return head_dim == 64 ? ValuEngine<KV, 64, 1, false>::kTile : ValuEngine<KV, 128, 1, false>::kTile;
}

}  // namespace

int rows_per_segment(int path, int kv_dtype, int n) {
  if (path == FD_PATH_MFMA) {
    for (int r = MfmaEngine<false, false>::kMaxRows; r > 1; --r)
      if (n % r == 0) return r;
    return 1;
  }
  if (kv_dtype != FD_FP8_E4M3 && n % 4 == 0) return 4;
  if (n % 2 == 0) return 2;
  return 1;
}

int kernel_tile(int path, int kv_dtype, int head_dim) {
  if (path == FD_PATH_MFMA) return MfmaEngine<false, false>::kTile;
  if (kv_dtype == FD_FP8_E4M3) return valu_tile<uint8_t>(head_dim);
  if (kv_dtype == FD_BF16) return valu_tile<uint16_t>(head_dim);
  return valu_tile<float>(head_dim);
}

bool mfma_supported(int kv_dtype, int head_dim, int rows) {
  return (kv_dtype == FD_BF16 || kv_dtype == FD_FP8_E4M3) && head_dim == 128 && rows >= 4 &&
         rows <= MfmaEngine<false, false>::kMaxRows;
}

int resident_waves_per_cu(int path, int kv_dtype, int head_dim, int rows, int paged) {
  if (path == FD_PATH_MFMA) {
    if (kv_dtype == FD_FP8_E4M3)
      return paged ? occupancy_waves(partial_mfma_d128<true, true, FD_MODE_BALANCED>)
                   : occupancy_waves(partial_mfma_d128<false, true, FD_MODE_BALANCED>);
    return paged ? occupancy_waves(partial_mfma_d128<true, false, FD_MODE_BALANCED>)
                 : occupancy_waves(partial_mfma_d128<false, false, FD_MODE_BALANCED>);
  }
  if (kv_dtype == FD_FP8_E4M3) return valu_waves_kv<uint8_t>(head_dim, rows, paged);
  if (kv_dtype == FD_BF16) return valu_waves_kv<uint16_t>(head_dim, rows, paged);
  return valu_waves_kv<float>(head_dim, rows, paged);
}

hipError_t static_workspace(hipStream_t stream, void** ptr) {
  static std::mutex mu;
  static std::vector<void*> addr;   // per device: the device address of scratch
  // The GPU the stream belongs to (the current GPU for the null stream).
  int dev = 0;
  hipError_t se = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (se != hipSuccess) return se;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    // The lookup runs with `dev` current (each device has its own copy of
    // the array); the caller's current device is restored after it.
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_partial(const PartialLaunch& a, hipStream_t stream) {
  if (a.geo.mode == FD_MODE_BALANCED)
    return a.out ? launch_partial_mode<kModeBalancedFused>(a, stream)
                 : launch_partial_mode<FD_MODE_BALANCED>(a, stream);
  return launch_partial_mode<FD_MODE_SPLITS>(a, stream);
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream) {
  // Balanced mode with many segments of few records each (a large batch):
  // a wave per segment reads its records as whole rows. Otherwise the rows
  // of a segment are merged in parallel, row by row.
  const int segs = a.batch * a.geo.segs_per_seq;
  if (a.geo.mode == FD_MODE_BALANCED && segs >= kSegmentCombineMinSegs &&
      (a.geo.workers + segs - 1) / segs + 1 <= 8) {
    const dim3 grid((segs + kWaves - 1) / kWaves);
    if (a.head_dim == 64)
      hipLaunchKernelGGL((combine_segments<64>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((combine_segments<128>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (a.out_dtype == FD_BF16)
    return a.head_dim == 64 ? launch_combine_typed<uint16_t, 64>(a, stream)
                            : launch_combine_typed<uint16_t, 128>(a, stream);
  return a.head_dim == 64 ? launch_combine_typed<float, 64>(a, stream) : launch_combine_typed<float, 128>(a, stream);
}

}  // namespace fd
