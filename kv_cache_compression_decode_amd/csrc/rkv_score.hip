// Host launcher of the scoring pass (kernels in rkv_score_impl.h, one
// translation unit per cache dtype, head_dim and layout).
#include "rkv_score_impl.h"

namespace rkv {

hipError_t launch_score(const ScoreArgs& a, bool bf16, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  const int grid = units * a.max_chunks;
  if (grid == 0) return hipSuccess;
  const int rt1 = (a.gw + 15) / 16;
  const int rt2 = (a.gw + 2 + 15) / 16;
#define RKV_PICK(DT, D)                                                              \
  return a.g.paged ? dispatch_score_##DT##_d##D##_paged(a, grid, rt1, rt2, st)       \
                   : dispatch_score_##DT##_d##D##_contig(a, grid, rt1, rt2, st)
  if (bf16) {
    if (a.g.d == 64) RKV_PICK(bf16, 64);
    RKV_PICK(bf16, 128);
  }
  if (a.g.d == 64) RKV_PICK(f32, 64);
  RKV_PICK(f32, 128);
#undef RKV_PICK
}

}  // namespace rkv
