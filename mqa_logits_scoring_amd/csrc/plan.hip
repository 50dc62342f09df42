// The plan kernel: one workgroup per plan segment (plan_segment.h), plus the
// copy of a plan's windows for inspection.
#include "plan_segment.h"

namespace idx {

namespace {

__global__ void __launch_bounds__(kSortThreads) plan_kernel(const PlanParams P) {
  __shared__ PlanSmem sm;
  plan_segment(P, blockIdx.x, sm);
}

// A plan recorded for other dimensions is not read past its header: every
// window is then reported as [-1, -1).
__global__ void copy_windows_kernel(const unsigned char* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H,
                                    int32_t D, size_t off_start, size_t off_end, int32_t* ws, int32_t* we) {
  const int64_t n_rows = int64_t(B) * S_q;
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const PlanHeader* hdr = reinterpret_cast<const PlanHeader*>(plan);
  const bool ok = hdr->magic == kPlanMagic && hdr->B == B && hdr->S_q == S_q && hdr->S_k == S_k && hdr->H == H &&
                  hdr->D == D;
  ws[r] = ok ? reinterpret_cast<const int32_t*>(plan + off_start)[r] : -1;
  we[r] = ok ? reinterpret_cast<const int32_t*>(plan + off_end)[r] : -1;
}

}  // namespace

hipError_t launch_plan(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* offsets,
                       const int32_t* starts, const int32_t* ends, void* plan, hipStream_t stream) {
  PlanParams P{};
  P.B = B;
  P.S_q = S_q;
  P.S_k = S_k;
  P.H = H;
  P.D = D;
  P.offsets = offsets;
  P.starts = starts;
  P.ends = ends;
  P.plan = static_cast<unsigned char*>(plan);
  P.L = plan_layout(B, S_q, H);
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(plan_segments(B, S_q))), dim3(kSortThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_plan_paged(int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D, const int32_t* ctx,
                             void* plan, hipStream_t stream) {
  PlanParams P{};
  P.B = B;
  P.S_q = S_q;
  P.S_k = S_k;
  P.H = H;
  P.D = D;
  P.plan = static_cast<unsigned char*>(plan);
  P.L = plan_layout(B, S_q, H);
  P.ctx = ctx;
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(plan_segments(B, S_q))), dim3(kSortThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_plan_thd(int32_t n_seg, const int32_t* cu_q, const int32_t* cu_k, int32_t ratio, int32_t T_q,
                           int32_t m_total, int32_t H, int32_t D, void* plan, hipStream_t stream) {
  PlanParams P{};
  P.B = 1;
  P.S_q = T_q;
  P.S_k = m_total;
  P.H = H;
  P.D = D;
  P.plan = static_cast<unsigned char*>(plan);
  P.L = plan_layout(1, T_q, H);
  P.cu_q = cu_q;
  P.cu_k = cu_k;
  P.n_seg = n_seg;
  P.ratio = ratio;
  hipLaunchKernelGGL(plan_kernel, dim3(unsigned(plan_segments(1, T_q))), dim3(kSortThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_copy_windows(const void* plan, int32_t B, int32_t S_q, int32_t S_k, int32_t H, int32_t D,
                               int32_t* ws, int32_t* we, hipStream_t stream) {
  const PlanLayout L = plan_layout(B, S_q, H);
  const int threads = 256;
  const int64_t blocks = (L.n_rows + threads - 1) / threads;
  hipLaunchKernelGGL(copy_windows_kernel, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                     static_cast<const unsigned char*>(plan), B, S_q, S_k, H, D, L.off_start, L.off_end, ws, we);
  return hipGetLastError();
}

}  // namespace idx
