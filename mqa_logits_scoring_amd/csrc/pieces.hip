// Weighted-query pieces: qt = sum_h w_h q_h for every query row, written as
// kPieces e4m3 rows with E8M0 block scales (see internal.h).  One wave per
// row; in the encoder lane l owns elements 2l and 2l+1, so lanes 16b..16b+15
// hold the 32-element block b.  Element decoding follows the OCP 8-bit float and OCP
// Microscaling v1.0 definitions; the e4m3 encoder rounds to nearest even.
#include "internal.h"

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

// Q rows are read in 16-byte loads, a whole wave covering 1 KB per load: in
// load i lane l holds EPL consecutive elements d0 = (l % LPH) * EPL.. of head
// HPL * i + l / LPH.  Each lane accumulates w_h q_h over its heads; lanes that
// share d0 are then summed with xor shuffles (a fixed order), and the row's
// qt goes through LDS to the lane-owns-two-elements layout of the encoder.
template <int F>
struct PieceLoad {
  static constexpr int EPL = F == IDX_IN_MXFP4_E2M1 ? 32 : 16;  // elements per lane per load
  static constexpr int LPH = 128 / EPL;                         // lanes per head
  static constexpr int HPL = 64 / LPH;                          // heads per load
  static constexpr int NL = 64 / HPL;                           // loads per row
  static constexpr int ROWB = F == IDX_IN_MXFP4_E2M1 ? 64 * 64 : 64 * 128;  // Q bytes per row
};

template <int F, bool WBF>
__global__ void __launch_bounds__(256) pieces_kernel(const void* q, const void* q_scale, const void* w, int64_t n_rows,
                                                     unsigned char* pieces, uint32_t* pscales) {
  using P = PieceLoad<F>;
  __shared__ float qt_lds[4][128];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t row_raw = int64_t(blockIdx.x) * 4 + wid;
  const bool live = row_raw < n_rows;
  const int64_t row = live ? row_raw : n_rows - 1;  // every wave reaches the barrier
  const int sub = lane % P::LPH, hl = lane / P::LPH;
  const unsigned char* qrow = static_cast<const unsigned char*>(q) + row * P::ROWB + lane * 16;
  float acc[P::EPL];
#pragma unroll
  for (int e = 0; e < P::EPL; ++e) acc[e] = 0.f;
  uint4 raw[P::NL];
#pragma unroll
  for (int i = 0; i < P::NL; ++i) raw[i] = *reinterpret_cast<const uint4*>(qrow + i * 1024);
#pragma unroll
  for (int i = 0; i < P::NL; ++i) {
    const int64_t qh = row * 64 + P::HPL * i + hl;
    const float wh = WBF ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(w)[qh]) << 16)
                         : static_cast<const float*>(w)[qh];
    float sc = 1.f;
    if constexpr (F != IDX_IN_FP8_E4M3)
      sc = e8m0_value((static_cast<const uint32_t*>(q_scale)[qh] >> (8 * (sub * P::EPL / 32))) & 0xFFu);
    const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int e = 0; e < P::EPL; ++e) {
      float v;
      if constexpr (F == IDX_IN_MXFP4_E2M1)
        v = e2m1_value((wd[e / 8] >> (4 * (e % 8))) & 15u);
      else
        v = e4m3_value((wd[e / 4] >> (8 * (e % 4))) & 0xFFu);
      acc[e] = __builtin_fmaf(wh, v * sc, acc[e]);
    }
  }
#pragma unroll
  for (int o = P::LPH; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < P::EPL; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  if (hl == 0) {
#pragma unroll
    for (int e = 0; e < P::EPL; ++e) qt_lds[wid][sub * P::EPL + e] = acc[e];
  }
  __syncthreads();
  if (!live) return;
  const float a0 = qt_lds[wid][2 * lane], a1 = qt_lds[wid][2 * lane + 1];
  // pieces: each encodes the exact residual left by the ones before it
  float r0 = a0, r1 = a1;
  for (int p = 0; p < kPieces; ++p) {
    float m = __builtin_fmaxf(__builtin_fabsf(r0), __builtin_fabsf(r1));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
    const uint32_t mb = __float_as_uint(m);
    const uint32_t E = (mb >> 23) & 0xFFu;
    uint32_t sbyte = 127u, c0 = 0u, c1 = 0u;
    if (E >= 9u) {  // else the residual is below 2^-118: leave it (piece of zeros)
      // scale 2^k with k the smallest exponent for which |r| / 2^k <= 448
      const int k = int(E) - 127 - 8 + ((mb & 0x7FFFFFu) > 0x600000u ? 1 : 0);
      sbyte = uint32_t(127 + k);
      const float inv = __uint_as_float(uint32_t(127 - k) << 23);  // 2^-k (k in [-118, 120])
      const float sc = __uint_as_float(sbyte << 23);
      c0 = e4m3_code(r0 * inv);
      c1 = e4m3_code(r1 * inv);
      r0 -= e4m3_value(c0) * sc;  // exact: the decoded piece is within a factor 2 of r
      r1 -= e4m3_value(c1) * sc;
    }
    reinterpret_cast<uint16_t*>(pieces + (row * kPieces + p) * 128)[lane] = uint16_t(c0 | (c1 << 8));
    const uint32_t word = (__shfl(sbyte, 0)) | (__shfl(sbyte, 16) << 8) | (__shfl(sbyte, 32) << 16) |
                          (__shfl(sbyte, 48) << 24);
    if (lane == 0) pscales[row * kPieces + p] = word;
  }
}

}  // namespace

hipError_t launch_pieces(idx_in_t fmt, idx_fp_t w_dtype, const void* q, const void* q_scale, const void* w,
                         int64_t n_rows, unsigned char* pieces, uint32_t* pscales, hipStream_t stream) {
  const dim3 grid(unsigned((n_rows + 3) / 4)), block(256);
  const bool wb = w_dtype == IDX_BF16;
#define IDX_PIECES(F)                                                                                         \
  if (wb)                                                                                                     \
    hipLaunchKernelGGL((pieces_kernel<F, true>), grid, block, 0, stream, q, q_scale, w, n_rows, pieces, pscales); \
  else                                                                                                        \
    hipLaunchKernelGGL((pieces_kernel<F, false>), grid, block, 0, stream, q, q_scale, w, n_rows, pieces, pscales);
  switch (fmt) {
    case IDX_IN_FP8_E4M3: IDX_PIECES(IDX_IN_FP8_E4M3) break;
    case IDX_IN_MXFP8_E4M3: IDX_PIECES(IDX_IN_MXFP8_E4M3) break;
    case IDX_IN_MXFP4_E2M1: IDX_PIECES(IDX_IN_MXFP4_E2M1) break;
    default: return hipErrorInvalidValue;
  }
#undef IDX_PIECES
  return hipGetLastError();
}

}  // namespace idx
