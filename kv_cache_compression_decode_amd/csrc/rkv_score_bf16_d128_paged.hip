// Scoring kernels instantiated for bf16 caches, head_dim 128, paged layout.
#include "rkv_score_impl.h"

namespace rkv {
hipError_t dispatch_score_bf16_d128_paged(const ScoreArgs& a, int grid, int rt1, int rt2,
                                     hipStream_t st) {
  return dispatch_score_layout<true, true, 128>(a, grid, rt1, rt2, st);
}
}  // namespace rkv
