// K copied into MFMA fragment order (see internal.h): one thread per 16-byte
// chunk of the output, reading the matching chunk of a K row; then, for the
// formats that have them, the per-row K scales in block order.  The chunk
// offsets per lane half follow the operand placement of each format (the same
// CBASE / CSTRIDE the scoring kernel used to read rows directly).
#include "internal.h"

namespace idx {

namespace {

template <int ROWB, int CBASE, int CSTRIDE>
__global__ void __launch_bounds__(256) kfrag_kernel(const unsigned char* k, int64_t B, int64_t S_k, int64_t nblk,
                                                    unsigned char* kfrag) {
  constexpr int NV = ROWB / 32;  // 16-byte chunks per lane per block (LB / 16)
  const int64_t total = B * nblk * NV * 64;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int lane = int(i & 63);
  const int v = int((i >> 6) % NV);
  const int64_t bu = (i >> 6) / NV;  // b * nblk + u
  const int64_t b = bu / nblk, u = bu % nblk;
  const int c = lane & 31, g = lane >> 5;
  const int64_t row = u * 32 + c;
  uint4 x = make_uint4(0, 0, 0, 0);
  if (row < S_k) x = *reinterpret_cast<const uint4*>(k + (b * S_k + row) * ROWB + CBASE * g + CSTRIDE * v);
  reinterpret_cast<uint4*>(kfrag)[i] = x;
}

// Per-row K scales in block order (internal.h): one thread per output word.
// SHIFT: right shift of an MX word for lane half 1 (0 for the FP8 fp32 scale).
template <int SHIFT>
__global__ void __launch_bounds__(256) kscale_kernel(const uint32_t* ks, int64_t B, int64_t S_k, int64_t nblk,
                                                     uint32_t* out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= B * nblk * 64) return;
  const int lane = int(i & 63);
  const int64_t bu = i >> 6;
  const int64_t b = bu / nblk, u = bu % nblk;
  const int64_t col = u * 32 + (lane & 31);
  uint32_t w = col < S_k ? ks[b * S_k + col] : 0u;
  if (lane >= 32) w >>= SHIFT;
  out[i] = w;
}

}  // namespace

hipError_t launch_kfrag(idx_in_t fmt, const void* k, const void* k_scale, int64_t B, int64_t S_k,
                        unsigned char* kfrag, uint32_t* kscale, hipStream_t stream) {
  const int64_t nblk = (S_k + 31) / 32;
  const int rowb = row_bytes_of(fmt);
  const int64_t total = B * nblk * (rowb / 32) * 64;
  const dim3 grid(unsigned((total + 255) / 256)), block(256);
  const unsigned char* kk = static_cast<const unsigned char*>(k);
  switch (fmt) {
    case IDX_IN_BF16:
      hipLaunchKernelGGL((kfrag_kernel<256, 128, 16>), grid, block, 0, stream, kk, B, S_k, nblk, kfrag);
      break;
    case IDX_IN_FP8_E4M3:
    case IDX_IN_MXFP8_E4M3:
      hipLaunchKernelGGL((kfrag_kernel<128, 16, 32>), grid, block, 0, stream, kk, B, S_k, nblk, kfrag);
      break;
    case IDX_IN_MXFP4_E2M1:
      hipLaunchKernelGGL((kfrag_kernel<64, 32, 16>), grid, block, 0, stream, kk, B, S_k, nblk, kfrag);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !has_kscale(fmt)) return e;
  const dim3 sgrid(unsigned((B * nblk * 64 + 255) / 256));
  const uint32_t* ks = static_cast<const uint32_t*>(k_scale);
  switch (fmt) {
    case IDX_IN_FP8_E4M3:
      hipLaunchKernelGGL((kscale_kernel<0>), sgrid, block, 0, stream, ks, B, S_k, nblk, kscale);
      break;
    case IDX_IN_MXFP8_E4M3:
      hipLaunchKernelGGL((kscale_kernel<8>), sgrid, block, 0, stream, ks, B, S_k, nblk, kscale);
      break;
    case IDX_IN_MXFP4_E2M1:
      hipLaunchKernelGGL((kscale_kernel<16>), sgrid, block, 0, stream, ks, B, S_k, nblk, kscale);
      break;
    default:
      break;
  }
  return hipGetLastError();
}

}  // namespace idx
