// Scoring kernels instantiated for f32 caches, head_dim 128, contiguous layout.
#include "rkv_score_impl.h"

namespace rkv {
hipError_t dispatch_score_f32_d128_contig(const ScoreArgs& a, int grid, int rt1, int rt2,
                                     hipStream_t st) {
  return dispatch_score_layout<false, false, 128>(a, grid, rt1, rt2, st);
}
}  // namespace rkv
