// Scoring kernels for mxfp8 Q/K: every head count x weight type x output
// type x clean flag.
#include "score_kernel_gh.h"

namespace idx {

hipError_t launch_score_mxfp8(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                              hipStream_t stream) {
  return launch_score_fmt<IDX_IN_MXFP8_E4M3>(w_dtype, out_dtype, clean, a, stream);
}

}  // namespace idx
