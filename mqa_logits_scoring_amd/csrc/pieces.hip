// Weighted-query pieces: qt = sum_h w_h q_h for every query row, written as
// kPieces e4m3 rows with E8M0 block scales (see internal.h).  One wave per
// row; lane l owns elements 2l and 2l+1, so lanes 16b..16b+15 hold the
// 32-element block b.  Element decoding follows the OCP 8-bit float and OCP
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

template <int F, bool WBF>
__global__ void __launch_bounds__(256) pieces_kernel(const void* q, const void* q_scale, const void* w, int64_t n_rows,
                                                     unsigned char* pieces, uint32_t* pscales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int blk = lane >> 4;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll 16
  for (int h = 0; h < 64; ++h) {
    const int64_t qh = row * 64 + h;
    const float wh = WBF ? __uint_as_float(uint32_t(static_cast<const uint16_t*>(w)[qh]) << 16)
                         : static_cast<const float*>(w)[qh];
    float v0, v1;
    if constexpr (F == IDX_IN_MXFP4_E2M1) {
      const uint32_t byte = static_cast<const unsigned char*>(q)[qh * 64 + lane];
      v0 = e2m1_value(byte & 15u);
      v1 = e2m1_value(byte >> 4);
    } else {
      const uint32_t two = static_cast<const uint16_t*>(q)[qh * 64 + lane];
      v0 = e4m3_value(two & 0xFFu);
      v1 = e4m3_value(two >> 8);
    }
    if constexpr (F != IDX_IN_FP8_E4M3) {
      const float sc = e8m0_value((static_cast<const uint32_t*>(q_scale)[qh] >> (8 * blk)) & 0xFFu);
      v0 *= sc;
      v1 *= sc;
    }
    a0 = __builtin_fmaf(wh, v0, a0);
    a1 = __builtin_fmaf(wh, v1, a1);
  }
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
