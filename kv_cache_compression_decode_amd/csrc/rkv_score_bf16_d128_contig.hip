// Scoring kernels instantiated for bf16 caches, head_dim 128, contiguous layout.
#include "rkv_long_impl.h"
#include "rkv_step_impl.h"

namespace rkv {
hipError_t dispatch_score_bf16_d128_contig(const ScoreArgs& a, int grid, int rt1, int rt2,
                                     hipStream_t st) {
  return dispatch_score_layout<true, false, 128>(a, grid, rt1, rt2, st);
}
hipError_t dispatch_unit_bf16_d128_contig(const ScoreArgs& a, int units, int rt2, hipStream_t st) {
  return dispatch_unit<false, 128>(a, units, rt2, st);
}
hipError_t dispatch_step_bf16_d128_contig(const StepArgs& a, int units, int rt2, hipStream_t st) {
  return dispatch_step<false, 128>(a, units, rt2, st);
}
hipError_t dispatch_long_bf16_d128_contig(const ScoreArgs& a, int chunks, int rt2, hipStream_t st) {
  return dispatch_long<false, 128>(a, chunks, rt2, st);
}
}  // namespace rkv
