// Scoring kernels for mxfp4 Q/K: every weight type x output type x clean flag.
#include "score_kernel.h"

namespace idx {

hipError_t launch_score_mxfp4(idx_fp_t w_dtype, idx_fp_t out_dtype, bool clean, const ScoreArgs& a,
                             hipStream_t stream) {
  const bool wb = w_dtype == IDX_BF16, ob = out_dtype == IDX_BF16;
  if (wb) {
    if (ob) return clean ? launch_score_t<IDX_IN_MXFP4_E2M1, true, true, true>(a, stream)
                         : launch_score_t<IDX_IN_MXFP4_E2M1, true, true, false>(a, stream);
    return clean ? launch_score_t<IDX_IN_MXFP4_E2M1, true, false, true>(a, stream)
                 : launch_score_t<IDX_IN_MXFP4_E2M1, true, false, false>(a, stream);
  }
  if (ob) return clean ? launch_score_t<IDX_IN_MXFP4_E2M1, false, true, true>(a, stream)
                       : launch_score_t<IDX_IN_MXFP4_E2M1, false, true, false>(a, stream);
  return clean ? launch_score_t<IDX_IN_MXFP4_E2M1, false, false, true>(a, stream)
               : launch_score_t<IDX_IN_MXFP4_E2M1, false, false, false>(a, stream);
}

}  // namespace idx
