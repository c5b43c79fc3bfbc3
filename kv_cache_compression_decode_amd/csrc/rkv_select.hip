// Selection of the R-KV compression step: per triggered unit, keep the last
// `window` tokens and the budget - window highest-scoring other tokens (hotdry
// blog post, R-KV section: keep what is important and not redundant; R-KV
// project page, "How R-KV decides what to drop": budget and local window).
// Equal scores: the lower position is kept.  Output in ascending position.
//
// One workgroup per unit.  Scores map to order-preserving uint32 keys in LDS;
// an MSB-first 8-bit radix select finds the (budget - window)-th largest key
// t and how many keys equal to t are kept; two workgroup scans then emit the
// kept positions in order.
#include "rkv_device.h"
#include "rkv_launch.h"

namespace rkv {

namespace {

// Order-preserving map float -> uint32 (larger float, larger key); -0 -> +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive scan over the 256 threads of the workgroup.  `tmp` holds 4 ints.
__device__ __forceinline__ int block_incl_scan(int v, int* tmp) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += tmp[w];
  __syncthreads();
  return base + x;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int tmp[4];
  __shared__ int sh_digit, sh_gt;

  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  const int tid = threadIdx.x;
  const int cand = u.n - a.g.window;
  const int want = a.g.budget - a.g.window;
  const float* srow = a.scores + out_row(a.g, u) * a.score_stride;
  int32_t* krow = a.keep + out_row(a.g, u) * a.g.budget;

  for (int j = tid; j < cand; j += kThreads) keys[j] = order_key(srow[j]);
  __syncthreads();

  uint32_t prefix = 0u, mask = 0u;
  int r = want;                      // keys still to take at or below the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < cand; j += kThreads) {
      const uint32_t kk = keys[j];
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    const int c = hist[255 - tid];   // bins in descending digit order
    const int incl = block_incl_scan(c, tmp);
    if (incl >= r && incl - c < r) {
      sh_digit = 255 - tid;
      sh_gt = incl - c;
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    mask |= 0xFFu << shift;
    r -= sh_gt;
    __syncthreads();
  }
  // prefix = the want-th largest key; keep every larger key and the first r
  // equal ones in position order.
  const int per = (cand + kThreads - 1) / kThreads;
  const int lo = min(tid * per, cand), hi = min(lo + per, cand);
  int ceq = 0, cgt = 0;
  for (int j = lo; j < hi; ++j) {
    const uint32_t kk = keys[j];
    ceq += kk == prefix;
    cgt += kk > prefix;
  }
  const int eq_before = block_incl_scan(ceq, tmp) - ceq;
  const int take_eq = max(0, min(r - eq_before, ceq));
  const int nkeep = cgt + take_eq;
  int o = block_incl_scan(nkeep, tmp) - nkeep;
  int eqi = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t kk = keys[j];
    bool kp = kk > prefix;
    if (kk == prefix) {
      kp = eqi < r;
      ++eqi;
    }
    if (kp) krow[o++] = j;
  }
  for (int i = tid; i < a.g.window; i += kThreads) krow[want + i] = cand + i;
}

hipError_t prepare_select() {
  static hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               RKV_MAX_LEN * (int)sizeof(uint32_t));
  return once;
}

hipError_t launch_select(const SelectArgs& a, int max_len, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  if (units == 0) return hipSuccess;
  const size_t lds = (size_t)max_len * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kernel, dim3(units), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace rkv
