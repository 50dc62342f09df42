// Per-call preparation, one launch: the plan when the call builds it
// (plan_segment.h), K in MFMA fragment order, the per-row K scales in block
// order, and the weighted-query pieces, or for calls that accumulate FP8 /
// MXFP8 products exactly, Q and K converted to bf16 (all laid out in
// internal.h).  The jobs are independent, so their workgroups share one grid
// and overlap: the latency-bound plan and pieces workgroups come first, the
// bandwidth-bound copies fill the machine behind them.
//
// Element decoding follows the OCP 8-bit float and OCP Microscaling v1.0
// definitions; the e4m3 encoder of the pieces rounds to nearest even.
#include "plan_segment.h"

namespace idx {

namespace {

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;  // m * 2^-9
  return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float v = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : 0.5f * float(m);
  return (c & 8u) ? -v : v;
}

__device__ __forceinline__ float e8m0_value(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);  // 2^(e-127); 0 -> 2^-127
}

// |x| <= 448: nearest e4m3 code, ties to even (sign kept)
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float ax = __builtin_fabsf(x);
  uint32_t code;
  if (ax < 0.015625f) {  // below 2^-6: multiples of 2^-9 (8 * 2^-9 is the smallest normal, code 0x08)
    code = uint32_t(__float2int_rn(ax * 512.f));
  } else {
    uint32_t a = __float_as_uint(ax);
    a += 0x7FFFFu + ((a >> 20) & 1u);  // round the fraction to 3 bits, ties to even
    code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  }
  return sign | code;
}

// |x| < 4: nearest e2m1 code, ties to even (sign kept); the grid below 4 is
// {0, .5, 1, 1.5, 2, 3, 4}
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float ax = __builtin_fabsf(x);
  const uint32_t code = ax <= 0.25f ? 0u
                        : ax < 0.75f ? 1u
                        : ax <= 1.25f ? 2u
                        : ax < 1.75f ? 3u
                        : ax <= 2.5f ? 4u
                        : ax < 3.5f ? 5u
                        : 6u;
  return sign | code;
}

struct PrepArgs {
  // K reorder and K scales
  const unsigned char* k;
  const uint32_t* k_scale;
  int64_t B, S_k, nblk;
  FastDiv by_nblk, by_page;  // division by nblk and by the page size
  int32_t kgroup;             // K chunks (and K scale words) per thread, 1..kMaxGroup
  unsigned char* kfrag;
  uint32_t* kscale;
  // weighted-query pieces
  const void* q;
  const void* q_scale;
  const void* w;
  int64_t n_rows;
  unsigned char* pieces;
  uint32_t* pscales;
  // keys from a paged cache (k, k_scale unused then)
  bool paged;
  PagedK pk;
  // the plan, when built here
  PlanParams plan;
  // Q converted to bf16 ([n_rows, H, 128]), for calls that convert
  uint16_t* qconv;
  int32_t H;
  // workgroups of each job, in grid order: plan segments, pieces or Q
  // conversion, K chunks, K scales
  int64_t n_plan, n_pieces, n_qconv, n_kfrag, n_kscale;
};

// Row of the key source holding key `row` of batch (request) b, or -1 for
// none: row b * S_k + row of contiguous K, or for a paged cache the row of the
// request's page (page index clamped into the cache; nothing past the
// request's context, whose block-table entries are never read).
__device__ inline int64_t key_source_row(const PrepArgs& a, int64_t b, int64_t row) {
  if (row >= a.S_k) return -1;
  if (!a.paged) return b * a.S_k + row;
  int64_t n = a.pk.ctx[b];
  n = n < 0 ? 0 : (n > a.S_k ? a.S_k : n);
  if (row >= n) return -1;
  const uint32_t pi = a.by_page.div(uint32_t(row));  // row < S_k < 2^31
  int64_t page = a.pk.block_table[b * a.pk.max_pages + pi];
  page = page < 0 ? 0 : (page >= a.pk.num_pages ? a.pk.num_pages - 1 : page);
  return page * a.pk.page_size + (uint32_t(row) - pi * uint32_t(a.pk.page_size));
}

// Paged calls skip the 32-key blocks that lie wholly past a request's
// context: no window reaches them, so the scoring kernel stores nothing
// computed from them (it may read one block past a chunk's end, and those
// columns are never stored).  Contiguous K is copied whole.
__device__ inline bool block_unused(const PrepArgs& a, int64_t b, int64_t u) {
  if (!a.paged) return false;
  int64_t n = a.pk.ctx[b];
  n = n < 0 ? 0 : (n > a.S_k ? a.S_k : n);
  return u * 32 >= n;
}

// K chunks and scale words per thread at most: a thread issues all its loads
// before its stores, so the dependent reads of a paged gather (context, block
// table, cache row) overlap instead of queueing one after another.
constexpr int kMaxGroup = 8;

// One thread per 16-byte chunk of K in fragment order (kgroup of them per
// thread, 256 consecutive chunks apart), reading the matching chunk of a K
// row (offsets per lane half as the scoring kernel places d).
template <int ROWB, int CBASE, int CSTRIDE>
__device__ void kfrag_group(const PrepArgs& a, int64_t wg) {
  constexpr int NV = ROWB / 32;  // 16-byte chunks per lane per block
  const int64_t n = a.B * a.nblk * NV * 64;
  const unsigned char* base = a.paged ? a.pk.k_cache : a.k;
  uint4 x[kMaxGroup];
  int64_t at[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    at[j] = -1;
    x[j] = make_uint4(0, 0, 0, 0);
    const int64_t i = (wg * a.kgroup + j) * 256 + threadIdx.x;
    if (j >= a.kgroup || i >= n) continue;
    const int lane = int(i & 63);
    const int v = int((i >> 6) % NV);
    const uint32_t bu = uint32_t((i >> 6) / NV);  // b * nblk + u (< 2^32, checked on the host)
    const uint32_t b32 = a.by_nblk.div(bu);
    const int64_t b = b32, u = bu - b32 * uint32_t(a.nblk);
    if (block_unused(a, b, u)) continue;
    at[j] = i;
    const int c = lane & 31, g = lane >> 5;
    const int64_t src = key_source_row(a, b, u * 32 + c);
    if (src >= 0) x[j] = *reinterpret_cast<const uint4*>(base + src * ROWB + CBASE * g + CSTRIDE * v);
  }
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j)
    if (at[j] >= 0) reinterpret_cast<uint4*>(a.kfrag)[at[j]] = x[j];
}

// bf16 bits of a finite float, rounded to nearest even (exact for the
// converted e4m3 values: four significant bits, within bf16's range)
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Eight e4m3 codes (little-endian in `c`) times an E8M0 scale as eight bf16
// values, in order: the hardware decode at scale 1 is exact, the scale a
// multiply by a power of two.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c, float scale) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.f, false);
  const f2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.x, 1.f, true);
  const f2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.f, false);
  const f2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c.y, 1.f, true);
  auto pack = [&](f2 v) { return bf16_rne(v.x * scale) | (bf16_rne(v.y * scale) << 16); };
  return make_uint4(pack(a), pack(b), pack(d), pack(e));
}

// Q converted to bf16: one thread per 8 elements of one (row, head), its
// MX block scale folded in (FP8 Q has none).
template <int F>
__device__ void qconv_rows(const PrepArgs& a, int64_t wg) {
  const int64_t i = wg * 256 + threadIdx.x;
  if (i >= a.n_rows * a.H * 16) return;
  const int64_t qh = i >> 4;
  const int t = int(i & 15);
  const uint2 c = *reinterpret_cast<const uint2*>(static_cast<const unsigned char*>(a.q) + qh * 128 + 8 * t);
  float scale = 1.f;
  if constexpr (F == IDX_IN_MXFP8_E4M3)
    scale = e8m0_value((static_cast<const uint32_t*>(a.q_scale)[qh] >> (8 * (t >> 2))) & 0xFFu);
  reinterpret_cast<uint4*>(a.qconv)[i] = e4m3x8_to_bf16(c, scale);
}

// K converted to bf16 in the bf16 fragment order (KLayout<IDX_IN_BF16>): one
// thread per 16-byte chunk (kgroup of them per thread, as kfrag_group), that
// is 8 elements [64 g + 8 v, +8) of key row 32 u + c, MX block scale folded in.
template <int F>
__device__ void kconv_group(const PrepArgs& a, int64_t wg) {
  constexpr int NV = 8;  // 16-byte chunks per lane per block (256-byte bf16 rows)
  const int64_t n = a.B * a.nblk * NV * 64;
  const unsigned char* base = a.paged ? a.pk.k_cache : a.k;
  const uint32_t* sbase = a.paged ? a.pk.k_scale_cache : a.k_scale;
  uint2 x[kMaxGroup];
  float sc[kMaxGroup];
  int64_t at[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    at[j] = -1;
    x[j] = make_uint2(0, 0);
    sc[j] = 1.f;
    const int64_t i = (wg * a.kgroup + j) * 256 + threadIdx.x;
    if (j >= a.kgroup || i >= n) continue;
    const int lane = int(i & 63);
    const int v = int((i >> 6) % NV);
    const uint32_t bu = uint32_t((i >> 6) / NV);
    const uint32_t b32 = a.by_nblk.div(bu);
    const int64_t b = b32, u = bu - b32 * uint32_t(a.nblk);
    if (block_unused(a, b, u)) continue;
    at[j] = i;
    const int c = lane & 31, g = lane >> 5, e0 = 64 * g + 8 * v;
    const int64_t src = key_source_row(a, b, u * 32 + c);
    if (src >= 0) {
      x[j] = *reinterpret_cast<const uint2*>(base + src * 128 + e0);
      if constexpr (F == IDX_IN_MXFP8_E4M3) sc[j] = e8m0_value((sbase[src] >> (8 * (e0 >> 5))) & 0xFFu);
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j)
    if (at[j] >= 0) reinterpret_cast<uint4*>(a.kfrag)[at[j]] = e4m3x8_to_bf16(x[j], sc[j]);
}

// One thread per word of the K scales in block order (kgroup per thread, as
// above).  SHIFT: right shift of an MX word for lane half 1 (0 for the FP8
// fp32 scale).
template <int SHIFT>
__device__ void kscale_group(const PrepArgs& a, int64_t wg) {
  const int64_t n = a.B * a.nblk * 64;
  const uint32_t* base = a.paged ? a.pk.k_scale_cache : a.k_scale;
  uint32_t word[kMaxGroup];
  int64_t at[kMaxGroup];
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j) {
    at[j] = -1;
    word[j] = 0u;
    const int64_t i = (wg * a.kgroup + j) * 256 + threadIdx.x;
    if (j >= a.kgroup || i >= n) continue;
    const int lane = int(i & 63);
    const uint32_t bu = uint32_t(i >> 6);
    const uint32_t b32 = a.by_nblk.div(bu);
    const int64_t b = b32, u = bu - b32 * uint32_t(a.nblk);
    if (block_unused(a, b, u)) continue;
    at[j] = i;
    const int64_t src = key_source_row(a, b, u * 32 + (lane & 31));
    if (src >= 0) word[j] = base[src];
  }
#pragma unroll
  for (int j = 0; j < kMaxGroup; ++j)
    if (at[j] >= 0) a.kscale[at[j]] = (threadIdx.x & 32) ? word[j] >> SHIFT : word[j];
}

// Weighted query of one row, qt = sum_h w_h q_h, and its pieces, by one wave
// (a workgroup of 256 threads does 4 rows).  Lane l reads 16 bytes at
// l*16 + 1024*i of the row's 64 heads (i < 8 for e4m3, < 4 for e2m1): EPL
// consecutive elements d0 = (l % LPH) * EPL.. of head l / LPH + HPL * i.  Each
// lane decodes them exactly (the scaled converts with scale 1, then the E8M0
// block scale as a multiply, as the definition reads) and accumulates
// w_h * q_h over its heads.  A butterfly over the lanes that share d0 then
// leaves, stage by stage, half of the running sums in each lane
// (reduce-scatter; the order of every sum is fixed), until lane l holds
// qt[e], qt[e+1] with e = d0 + 2 * (l / LPH): the layout the encoder and the
// piece stores use.
template <int F>
struct PieceLoad {
  static constexpr bool E2M1 = F == IDX_IN_MXFP4_E2M1;
  static constexpr int EPL = E2M1 ? 32 : 16;  // elements per lane per load
  static constexpr int LPH = 128 / EPL;       // lanes per head (4 or 8)
  static constexpr int HPL = 64 / LPH;        // heads per load (16 or 8)
  static constexpr int NLW = 64 / HPL;        // loads per lane (4 or 8)
  static constexpr int HB = E2M1 ? 64 : 128;  // Q bytes per head
};

// x from lane l ^ 8 (a rotation by 8 inside each row of 16 lanes)
__device__ __forceinline__ float xor8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
// x from lane l ^ 4 (swizzle inside each group of 32 lanes)
__device__ __forceinline__ float xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}
// x from lane l ^ 1
__device__ __forceinline__ float xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_swap32(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_swap16(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

template <int F, bool WBF>
__device__ void pieces_rows(const PrepArgs& a, int64_t wg) {
  using P = PieceLoad<F>;
  using PF = PieceFmt<F>;
  constexpr bool E2M1 = P::E2M1;
  const int lane = threadIdx.x & 63;
  const int64_t row = wg * 4 + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  const int sub = lane % P::LPH, hl = lane / P::LPH;
  const int blk = sub * P::EPL / 32;  // the lane's 32-element block
  const unsigned char* qrow = static_cast<const unsigned char*>(a.q) + row * (64 * P::HB);
  uint4 raw[P::NLW];
#pragma unroll
  for (int i = 0; i < P::NLW; ++i) raw[i] = *reinterpret_cast<const uint4*>(qrow + i * 1024 + lane * 16);
  float acc[P::EPL];
#pragma unroll
  for (int e = 0; e < P::EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < P::NLW; ++i) {
    const int64_t qh = row * 64 + P::HPL * i + hl;
    const float wh = WBF ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.w)[qh]) << 16)
                         : static_cast<const float*>(a.w)[qh];
    float sc = 1.f;
    if constexpr (F != IDX_IN_FP8_E4M3)
      sc = e8m0_value((static_cast<const uint32_t*>(a.q_scale)[qh] >> (8 * blk)) & 0xFFu);
    const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
    typedef float f2 __attribute__((ext_vector_type(2)));
    auto add2 = [&](int e, f2 v) {
      acc[e] = __builtin_fmaf(wh, v.x * sc, acc[e]);
      acc[e + 1] = __builtin_fmaf(wh, v.y * sc, acc[e + 1]);
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (E2M1) {  // byte s of the word: elements 8k + 2s (low nibble), 8k + 2s + 1
        add2(8 * k + 0, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[k], 1.f, 0));
        add2(8 * k + 2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[k], 1.f, 1));
        add2(8 * k + 4, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[k], 1.f, 2));
        add2(8 * k + 6, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[k], 1.f, 3));
      } else {  // bytes 0-1 and 2-3 of the word: elements 4k.. 4k + 3
        add2(4 * k + 0, __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[k], 1.f, false));
        add2(4 * k + 2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(wd[k], 1.f, true));
      }
    }
  }
  // reduce-scatter over the lanes sharing d0 (lane bits above log2(LPH)):
  // each stage halves the sums a lane keeps, splitting the element index on
  // its highest remaining bit, so the two left are adjacent elements
  float r0, r1;
  {
    float v32[P::EPL / 2];  // after lane ^ 32: element j + (EPL/2) * bit5
#pragma unroll
    for (int j = 0; j < P::EPL / 2; ++j) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j]), __float_as_uint(acc[j + P::EPL / 2]),
                                                       false, false);
      v32[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    constexpr int N16 = P::EPL / 4;
    float v16[N16];  // after lane ^ 16
#pragma unroll
    for (int j = 0; j < N16; ++j) {
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v32[j]), __float_as_uint(v32[j + N16]), false,
                                                       false);
      v16[j] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    constexpr int N8 = P::EPL / 8;
    const bool b3 = (lane & 8) != 0;
    float v8[N8];  // after lane ^ 8
#pragma unroll
    for (int j = 0; j < N8; ++j) {
      const float keep = b3 ? v16[j + N8] : v16[j], send = b3 ? v16[j] : v16[j + N8];
      v8[j] = keep + xor8(send);
    }
    if constexpr (E2M1) {
      const bool b2 = (lane & 4) != 0;
      float v4[2];  // after lane ^ 4
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float keep = b2 ? v8[j + 2] : v8[j], send = b2 ? v8[j] : v8[j + 2];
        v4[j] = keep + xor4(send);
      }
      r0 = v4[0];
      r1 = v4[1];
    } else {
      r0 = v8[0];
      r1 = v8[1];
    }
  }
  // lane holds elements e0 = d0 + 2 * hl and e0 + 1
  const int e0 = sub * P::EPL + 2 * hl;
  // pieces: each encodes the exact residual left by the ones before it; the
  // block maximum runs over the 16 lanes of the lane's 32-element block
  for (int p = 0; p < PF::N; ++p) {
    float m = __builtin_fmaxf(__builtin_fabsf(r0), __builtin_fabsf(r1));
    if constexpr (E2M1) {
      m = __builtin_fmaxf(m, xor4(m));
    } else {
      m = __builtin_fmaxf(m, xor1(m));
    }
    m = __builtin_fmaxf(m, xor8(m));
    m = max_swap16(m);
    m = max_swap32(m);
    const uint32_t mb = __float_as_uint(m);
    const uint32_t E = (mb >> 23) & 0xFFu;
    uint32_t sbyte = 127u, c0 = 0u, c1 = 0u;
    if (E >= 9u) {  // else the residual is below 2^-118: leave it (piece of zeros)
      // e4m3: scale 2^k with k the smallest exponent for which |r| / 2^k <= 448;
      // e2m1: k = e - 1 for |r|max = 1.f 2^e, so |r| / 2^k < 4
      const int k = E2M1 ? int(E) - 128 : int(E) - 127 - 8 + ((mb & 0x7FFFFFu) > 0x600000u ? 1 : 0);
      sbyte = uint32_t(127 + k);
      const float inv = __uint_as_float(uint32_t(127 - k) << 23);  // 2^-k (k in [-119, 126])
      const float scl = __uint_as_float(sbyte << 23);
      if constexpr (E2M1) {
        c0 = e2m1_code(r0 * inv);
        c1 = e2m1_code(r1 * inv);
        r0 -= e2m1_value(c0) * scl;  // exact: the decoded piece is 0 or within a factor 2 of r
        r1 -= e2m1_value(c1) * scl;
      } else {
        c0 = e4m3_code(r0 * inv);
        c1 = e4m3_code(r1 * inv);
        r0 -= e4m3_value(c0) * scl;  // exact: the decoded piece is within a factor 2 of r
        r1 -= e4m3_value(c1) * scl;
      }
    }
    unsigned char* dst = a.pieces + row * kPieceRowBytes + p * PF::BYTES;
    if constexpr (E2M1)
      dst[e0 / 2] = uint8_t(c0 | (c1 << 4));  // elements e0 (low nibble) and e0 + 1
    else
      reinterpret_cast<uint16_t*>(dst)[e0 / 2] = uint16_t(c0 | (c1 << 8));
    // block b's byte from its first lane (sub = b * 32 / EPL, hl = 0)
    constexpr int LPB = 32 / P::EPL;  // lanes of sub per block (1 or 2)
    const uint32_t word = uint32_t(__builtin_amdgcn_readlane(int(sbyte), 0)) |
                          (uint32_t(__builtin_amdgcn_readlane(int(sbyte), 1 * LPB)) << 8) |
                          (uint32_t(__builtin_amdgcn_readlane(int(sbyte), 2 * LPB)) << 16) |
                          (uint32_t(__builtin_amdgcn_readlane(int(sbyte), 3 * LPB)) << 24);
    if (lane == 0) a.pscales[row * kPieceSlots + p] = word;
  }
}

// CONV: Q and K of an FP8 / MXFP8 call converted to bf16 (no pieces; the
// FP8 row scales still go to block order).
template <int F, bool WBF, bool CONV>
__global__ void __launch_bounds__(256) prepare_kernel(const PrepArgs a) {
  using L = KLayout<F>;
  __shared__ union {
    PlanSmem plan;
  } sm;
  int64_t bid = blockIdx.x;
  if (bid < a.n_plan) {
    plan_segment(a.plan, bid, sm.plan);
    return;
  }
  bid -= a.n_plan;
  if constexpr (CONV) {
    if (bid < a.n_qconv) {
      qconv_rows<F>(a, bid);
      return;
    }
    bid -= a.n_qconv;
    if (bid < a.n_kfrag) {
      kconv_group<F>(a, bid);
      return;
    }
    bid -= a.n_kfrag;
    if constexpr (F == IDX_IN_FP8_E4M3) kscale_group<0>(a, bid);
  } else {
    if constexpr (F != IDX_IN_BF16) {
      if (bid < a.n_pieces) {
        pieces_rows<F, WBF>(a, bid);
        return;
      }
      bid -= a.n_pieces;
    }
    if (bid < a.n_kfrag) {
      kfrag_group<L::ROWB, L::CBASE, L::CSTRIDE>(a, bid);
      return;
    }
    bid -= a.n_kfrag;
    if constexpr (F != IDX_IN_BF16) kscale_group<L::SHIFT>(a, bid);
  }
}

template <int F, bool WBF, bool CONV = false>
hipError_t launch(const PrepArgs& a, hipStream_t stream) {
  const int64_t grid = a.n_plan + a.n_pieces + a.n_qconv + a.n_kfrag + a.n_kscale;
  if (grid == 0) return hipSuccess;  // e.g. BF16 keys read from a paged cache, plan given
  hipLaunchKernelGGL((prepare_kernel<F, WBF, CONV>), dim3(unsigned(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(idx_in_t fmt, bool convert, int H, idx_fp_t w_dtype, const void* k, const void* k_scale,
                          int64_t B, int64_t S_k, unsigned char* kfrag, uint32_t* kscale, const void* q,
                          const void* q_scale, const void* w, int64_t n_rows, unsigned char* pieces,
                          uint32_t* pscales, uint16_t* qconv, const PlanBuild* build, const PagedK* paged,
                          hipStream_t stream) {
  PrepArgs a{};
  if (paged != nullptr) {
    a.paged = true;
    a.pk = *paged;
  }
  if (build != nullptr) {
    a.plan = PlanParams{};
    a.plan.B = build->B;
    a.plan.S_q = build->S_q;
    a.plan.S_k = build->S_k;
    a.plan.H = build->H;
    a.plan.D = build->D;
    a.plan.offsets = build->offsets;
    a.plan.starts = build->starts;
    a.plan.ends = build->ends;
    a.plan.ctx = build->ctx;
    a.plan.plan = build->plan;
    a.plan.L = plan_layout(build->B, build->S_q, build->H);
    a.n_plan = plan_segments(build->B, build->S_q);
  }
  a.k = static_cast<const unsigned char*>(k);
  a.k_scale = static_cast<const uint32_t*>(k_scale);
  a.B = B;
  a.S_k = S_k;
  a.nblk = (S_k + 31) / 32;
  if (B * a.nblk >= (int64_t(1) << 32)) return hipErrorInvalidValue;  // block indices are 32-bit
  a.by_nblk = FastDiv::make(uint32_t(a.nblk));
  a.by_page = FastDiv::make(paged != nullptr ? uint32_t(paged->page_size) : 1u);
  a.kfrag = kfrag;
  a.kscale = kscale;
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.n_rows = n_rows;
  a.pieces = pieces;
  a.pscales = pscales;
  a.qconv = qconv;
  a.H = H;
  const Exec x{convert ? (fmt == IDX_IN_FP8_E4M3 ? kInBF16RowScale : int(IDX_IN_BF16)) : int(fmt), convert};
  if (convert && fmt != IDX_IN_FP8_E4M3 && fmt != IDX_IN_MXFP8_E4M3) return hipErrorInvalidValue;
  const bool scaled = has_kscale(x.kf);
  a.n_pieces = pieces != nullptr ? (n_rows + 3) / 4 : 0;  // only 64-head calls of the formats with pieces
  a.n_qconv = convert ? (n_rows * H * 16 + 255) / 256 : 0;
  // several chunks per thread only when that still leaves at least 2048
  // workgroups of K copy
  const bool copy_k = paged == nullptr || !paged->skip_gather;
  const int64_t n_chunks = copy_k ? B * a.nblk * (row_bytes_of(x.kf) / 32) * 64 : 0;
  const int64_t per_wg = 256 * 2048;
  a.kgroup = int32_t(n_chunks / per_wg < 1 ? 1 : (n_chunks / per_wg > kMaxGroup ? kMaxGroup : n_chunks / per_wg));
  const int64_t span = 256 * int64_t(a.kgroup);
  a.n_kfrag = (n_chunks + span - 1) / span;
  a.n_kscale = scaled && copy_k ? (B * a.nblk * 64 + span - 1) / span : 0;
  if (a.n_plan + a.n_pieces + a.n_qconv + a.n_kfrag + a.n_kscale > (int64_t(1) << 31) - 1)
    return hipErrorInvalidValue;
  const bool wb = w_dtype == IDX_BF16;
  if (convert)  // the weights are not read
    return fmt == IDX_IN_FP8_E4M3 ? launch<IDX_IN_FP8_E4M3, false, true>(a, stream)
                                  : launch<IDX_IN_MXFP8_E4M3, false, true>(a, stream);
  switch (fmt) {
    case IDX_IN_BF16: return launch<IDX_IN_BF16, false>(a, stream);
    case IDX_IN_FP8_E4M3: return wb ? launch<IDX_IN_FP8_E4M3, true>(a, stream) : launch<IDX_IN_FP8_E4M3, false>(a, stream);
    case IDX_IN_MXFP8_E4M3:
      return wb ? launch<IDX_IN_MXFP8_E4M3, true>(a, stream) : launch<IDX_IN_MXFP8_E4M3, false>(a, stream);
    case IDX_IN_MXFP4_E2M1:
      return wb ? launch<IDX_IN_MXFP4_E2M1, true>(a, stream) : launch<IDX_IN_MXFP4_E2M1, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace idx
