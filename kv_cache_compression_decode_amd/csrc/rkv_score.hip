// Host launcher of the scoring pass (kernels in rkv_score_impl.h, one
// translation unit per cache dtype and head_dim).
#include "rkv_score_impl.h"

namespace rkv {

hipError_t launch_score(const ScoreArgs& a, bool bf16, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  const int grid = units * a.max_chunks;
  if (grid == 0) return hipSuccess;
  const int rt1 = (a.gw + 15) / 16;
  const int rt2 = (a.gw + 2 + 15) / 16;
  if (bf16)
    return a.g.d == 64 ? dispatch_score_bf16_d64(a, grid, rt1, rt2, st)
                       : dispatch_score_bf16_d128(a, grid, rt1, rt2, st);
  return a.g.d == 64 ? dispatch_score_f32_d64(a, grid, rt1, rt2, st)
                     : dispatch_score_f32_d128(a, grid, rt1, rt2, st);
}

}  // namespace rkv
