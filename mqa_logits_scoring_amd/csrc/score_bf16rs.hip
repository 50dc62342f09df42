// Scoring kernels for FP8 inputs accumulated exactly: Q and K converted to
// bf16 by the preparation, the per-row K scale applied after the head-sum.
#include "score_kernel_gh.h"

namespace idx {

hipError_t launch_score_bf16rs(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                               hipStream_t stream) {
  return launch_score_fmt<kInBF16RowScale>(w_dtype, out_dtype, clean, a, stream);
}

}  // namespace idx
