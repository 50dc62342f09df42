/*
 * idx_peak.h - matrix-core throughput probe for gfx950 (libidx_peak.so).
 *
 * A measurement aid beside the scoring library, not part of the scoring path:
 * bench.py uses it to re-measure on the machine the MFMA peaks that the
 * scoring kernels' roofline fractions are quoted against (the published
 * MI355X figures are dense bf16 2.5 PFLOP/s, fp8 5.0 and fp4 10.1).
 */
#ifndef IDX_PEAK_H
#define IDX_PEAK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The MFMA shapes the scoring kernels issue. */
enum {
  IDX_PEAK_BF16_32X32X16 = 0,   /* v_mfma_f32_32x32x16_bf16                     */
  IDX_PEAK_FP8_32X32X64 = 1,    /* v_mfma_scale_f32_32x32x64_f8f6f4, e4m3       */
  IDX_PEAK_FP8_16X16X128 = 2,   /* v_mfma_scale_f32_16x16x128_f8f6f4, e4m3      */
  IDX_PEAK_FP4_32X32X64 = 3,    /* v_mfma_scale_f32_32x32x64_f8f6f4, e2m1       */
  IDX_PEAK_FP4_16X16X128 = 4    /* v_mfma_scale_f32_16x16x128_f8f6f4, e2m1      */
};

/* FLOP of one MFMA of `kind` (2 * M * N * K); 0 for an unknown kind. */
double idx_peak_flop_per_mfma(int32_t kind);

/*
 * Enqueue on `stream` (a hipStream_t, NULL = default) `groups` workgroups of
 * 4 waves; every wave issues iters x 8 independent MFMAs of `kind` on register
 * operands (pseudo-random codes, or zeros when `zero` is nonzero) and writes
 * one float per thread to `out` (device memory of groups * 256 floats, owned
 * by the caller).  Total FLOP = groups * 4 * iters * 8 * idx_peak_flop_per_mfma.
 * Returns 0, 1 for invalid arguments (nothing enqueued), 2 for an unknown
 * kind, 4 for a launch failure.
 */
int32_t idx_peak_mfma(int32_t kind, int32_t groups, int32_t iters, int32_t zero, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IDX_PEAK_H */
