// MFMA throughput probe for gfx950: a measurement aid that stands beside the
// scoring library (include/idx_peak.h), used to re-measure on the machine the
// matrix-core peaks that the scoring kernels' roofline fractions are quoted
// against.  Nothing in the scoring path calls it.
//
// Every wave issues `iters` rounds of 8 independent MFMAs of one shape on
// register operands (8 accumulators, so the matrix pipe never waits on a
// dependency), then writes the sum of its accumulators so that none of the
// work can be dropped.  Operands are either pseudo-random codes (the power
// draw of real data) or zeros.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/idx_peak.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // integer hash (lowbias32, C. Wellons)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <int KIND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
    peak_kernel(int iters, int zero, float* out) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  // 8-bit codes with exponent fields below the top one (no e4m3 NaN), bf16
  // values in [1, 2) with random mantissas; all zero when asked
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t r = mix(gid * 8u + uint32_t(e) + 1u);
    w[e] = zero ? 0u : (KIND == IDX_PEAK_BF16_32X32X16 ? ((r & 0x007F007Fu) | 0x3F803F80u) : (r & 0x77777777u));
  }
  constexpr bool BIG = KIND == IDX_PEAK_BF16_32X32X16 || KIND == IDX_PEAK_FP8_32X32X64 || KIND == IDX_PEAK_FP4_32X32X64;
  typedef typename std::conditional<BIG, f32x16, f32x4>::type acc_t;
  // distinct starting values, so no two accumulator chains are the same
  // computation the compiler could merge
  acc_t acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = acc_t{} + float(i + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == IDX_PEAK_BF16_32X32X16) {
        bf16x8 a, b;
        __builtin_memcpy(&a, &w[0], 16);
        __builtin_memcpy(&b, &w[4], 16);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      } else {
        const i32x8 a = {int(w[0]), int(w[1]), int(w[2]), int(w[3]), int(w[4]), int(w[5]), int(w[6]), int(w[7])};
        const i32x8 b = {int(w[7]), int(w[6]), int(w[5]), int(w[4]), int(w[3]), int(w[2]), int(w[1]), int(w[0])};
        constexpr int CODE = (KIND == IDX_PEAK_FP4_32X32X64 || KIND == IDX_PEAK_FP4_16X16X128) ? 4 : 0;
        if constexpr (BIG)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], CODE, CODE, 0, 127, 0, 127);
        else
          acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], CODE, CODE, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < int(sizeof(acc_t) / 4); ++r) s += acc[i][r];
  out[gid] = s;
}

template <int KIND>
hipError_t launch(int groups, int iters, int zero, float* out, hipStream_t stream) {
  hipLaunchKernelGGL((peak_kernel<KIND>), dim3(unsigned(groups)), dim3(256), 0, stream, iters, zero, out);
  return hipGetLastError();
}

}  // namespace

extern "C" {

double idx_peak_flop_per_mfma(int32_t kind) {
  switch (kind) {
    case IDX_PEAK_BF16_32X32X16: return 2.0 * 32 * 32 * 16;
    case IDX_PEAK_FP8_32X32X64:
    case IDX_PEAK_FP4_32X32X64: return 2.0 * 32 * 32 * 64;
    case IDX_PEAK_FP8_16X16X128:
    case IDX_PEAK_FP4_16X16X128: return 2.0 * 16 * 16 * 128;
  }
  return 0.0;
}

int32_t idx_peak_mfma(int32_t kind, int32_t groups, int32_t iters, int32_t zero, float* out, void* stream) {
  if (groups <= 0 || iters <= 0 || out == nullptr) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case IDX_PEAK_BF16_32X32X16: e = launch<IDX_PEAK_BF16_32X32X16>(groups, iters, zero, out, s); break;
    case IDX_PEAK_FP8_32X32X64: e = launch<IDX_PEAK_FP8_32X32X64>(groups, iters, zero, out, s); break;
    case IDX_PEAK_FP8_16X16X128: e = launch<IDX_PEAK_FP8_16X16X128>(groups, iters, zero, out, s); break;
    case IDX_PEAK_FP4_32X32X64: e = launch<IDX_PEAK_FP4_32X32X64>(groups, iters, zero, out, s); break;
    case IDX_PEAK_FP4_16X16X128: e = launch<IDX_PEAK_FP4_16X16X128>(groups, iters, zero, out, s); break;
    default: return 2;
  }
  return e == hipSuccess ? 0 : 4;
}

}  // extern "C"
