// Workgroup-wide selection over scores staged in LDS, shared by the select
// kernel and the fused step kernel.  Per unit: keep the last `window`
// tokens and the budget - window highest-scoring others (hotdry blog post,
// R-KV section: keep what is important and not redundant; R-KV project page,
// "How R-KV decides what to drop": budget and local window); equal scores
// keep the lower position; output in ascending position.
//
// Scores are mapped to order-preserving uint32 keys; an MSB-first 8-bit
// radix select finds the (budget - window)-th largest key t and how many keys
// equal to t are kept; two workgroup scans emit the kept positions in order.
#pragma once

#include "rkv_device.h"

namespace rkv {

// Order-preserving map float -> uint32 (larger float, larger key); -0 -> +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Shared scratch of the selection (besides the keys).
template <int THREADS>
struct SelectShared {
  int hist[256];
  int tmp[THREADS / kWave];
  int digit, above;
};

// Inclusive scan over the workgroup.
template <int THREADS>
__device__ __forceinline__ int block_incl_scan(int v, int* tmp) {
  constexpr int W = THREADS / kWave;
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
#pragma unroll
  for (int w = 0; w < W; ++w)
    if (w < wave) base += tmp[w];
  __syncthreads();
  return base + x;
}

// keys[0, cand) hold order keys of the candidates; writes keep[0, budget)
// (global or LDS) and returns nothing.  All THREADS threads call it.
template <int THREADS, typename OutFn>
__device__ __forceinline__ void block_select(const uint32_t* keys, int cand, int want, int window,
                                             SelectShared<THREADS>& sh, OutFn out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u;
  int r = want;                      // keys still to take at or below the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += THREADS) sh.hist[b] = 0;
    __syncthreads();
    for (int j = tid; j < cand; j += THREADS) {
      const uint32_t kk = keys[j];
      if ((kk & mask) == prefix) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    const int c = tid < 256 ? sh.hist[255 - tid] : 0;   // bins in descending digit order
    const int incl = block_incl_scan<THREADS>(c, sh.tmp);
    if (tid < 256 && incl >= r && incl - c < r) {
      sh.digit = 255 - tid;
      sh.above = incl - c;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    mask |= 0xFFu << shift;
    r -= sh.above;
    __syncthreads();
  }
  // prefix = the want-th largest key; keep every larger key and the first r
  // equal ones in position order.
  const int per = (cand + THREADS - 1) / THREADS;
  const int lo = min(tid * per, cand), hi = min(lo + per, cand);
  int ceq = 0, cgt = 0;
  for (int j = lo; j < hi; ++j) {
    const uint32_t kk = keys[j];
    ceq += kk == prefix;
    cgt += kk > prefix;
  }
  const int eq_before = block_incl_scan<THREADS>(ceq, sh.tmp) - ceq;
  const int take_eq = max(0, min(r - eq_before, ceq));
  const int nkeep = cgt + take_eq;
  int o = block_incl_scan<THREADS>(nkeep, sh.tmp) - nkeep;
  int eqi = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t kk = keys[j];
    bool kp = kk > prefix;
    if (kk == prefix) {
      kp = eqi < r;
      ++eqi;
    }
    if (kp) out(o++, j);
  }
  for (int i = tid; i < window; i += THREADS) out(want + i, cand + i);
}

}  // namespace rkv
