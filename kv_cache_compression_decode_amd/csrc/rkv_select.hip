// Selection kernel of the R-KV compression step (rule and method in
// rkv_select_impl.h): one workgroup per triggered unit -- or, with head-shared
// selection, per (sequence, layer), ranking by the float32 sum of the heads'
// scores (head 0 first) and writing the keep row of every head.  The
// candidates' order keys are staged in LDS; every radix pass walks them all,
// so long units take 1024 threads, short ones 256.
#include "rkv_launch.h"
#include "rkv_select_impl.h"

namespace rkv {

template <int T>
__global__ __launch_bounds__(T) void select_kernel(SelectArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ SelectShared<T> sh;

  const int heads = a.g.shared ? a.g.hkv : 1;   // score rows ranked together
  const Unit u = decode_unit(a.g, a.tt, blockIdx.x * heads);   // head 0 when shared
  if (u.n == 0) return;   // past the device table's count
  if (step_aborted(a.status)) return;   // the step failed a device check: keep rows untouched
  const int cand = u.n - a.g.window;
  const int want = a.g.budget - a.g.window;
  const float* srow = a.scores + out_row(a.g, u) * a.score_stride;
  int32_t* krow = a.keep + out_row(a.g, u) * a.g.budget;

  for (int j = threadIdx.x; j < cand; j += T) {
    float sc = srow[j];
    for (int h = 1; h < heads; ++h) sc += srow[(int64_t)h * a.score_stride + j];
    keys[j] = order_key(sc);
  }
  block_select_init(sh);
  __syncthreads();
  block_select<T, 0>(
      keys, cand, want, a.g.window, sh,
      [&](int i, int pos) {
        for (int h = 0; h < heads; ++h) krow[(int64_t)h * a.g.budget + i] = pos;
      },
      [](int) {});
}

// 1024 threads from this many keys (measured: 9 vs 12 us at 1152 keys per unit,
// 10 vs 15 at 2176, 50 vs 74 at 4352 for the paged 2048-unit batch)
constexpr int kSelectWideFrom = 1024;

hipError_t prepare_select() {
  static hipError_t once = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<kThreads>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       RKV_MAX_LEN * (int)sizeof(uint32_t));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<1024>),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               RKV_MAX_LEN * (int)sizeof(uint32_t));
  }();
  return once;
}

hipError_t launch_select(const SelectArgs& a, int max_len, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * (a.g.shared ? 1 : a.g.hkv);
  if (units == 0) return hipSuccess;
  const size_t lds = (size_t)max_len * sizeof(uint32_t);
  if (max_len >= kSelectWideFrom)
    hipLaunchKernelGGL(select_kernel<1024>, dim3(units), dim3(1024), lds, st, a);
  else
    hipLaunchKernelGGL(select_kernel<kThreads>, dim3(units), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace rkv
