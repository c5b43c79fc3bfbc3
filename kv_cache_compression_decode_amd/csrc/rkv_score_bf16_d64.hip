// Scoring kernels instantiated for bf16 caches with head_dim 64.
#include "rkv_score_impl.h"

namespace rkv {
hipError_t dispatch_score_bf16_d64(const ScoreArgs& a, int grid, int rt1, int rt2, hipStream_t st) {
  return dispatch_score<true, 64>(a, grid, rt1, rt2, st);
}
}  // namespace rkv
