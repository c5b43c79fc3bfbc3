// Workgroup-wide selection over scores staged in LDS, shared by the select
// kernel and the fused step kernel.  Per unit: keep the last `window`
// tokens and the budget - window highest-scoring others (hotdry blog post,
// R-KV section: keep what is important and not redundant; R-KV project page,
// "How R-KV decides what to drop": budget and local window); equal scores
// keep the lower position; output in ascending position.
//
// Scores are mapped to order-preserving uint32 keys; an MSB-first 8-bit
// radix select finds the (budget - window)-th largest key t and how many keys
// equal to t are kept; one workgroup scan then gives every thread the output
// offset of its contiguous run of positions.  Each radix pass costs two
// barriers: one after the histogram, one after wave 0 has found the digit
// (the other waves clear the next pass's histogram meanwhile).
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
  __attribute__((aligned(16))) int hist[2][256];
  int tot[THREADS / kWave];
  int digit, above;
};

// Inclusive scan over the 64 lanes of a wave: DPP row shifts give the scan
// within each row of 16 lanes, then the row totals are added in.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int lane = threadIdx.x & (kWave - 1);
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
}

// Exclusive scan over the workgroup (one barrier).  Called once per
// workgroup lifetime: `tot` is not reused.
template <int THREADS>
__device__ __forceinline__ int block_excl_scan(int v, int* tot) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) tot[wave] = incl;
  lds_barrier();
  int base = 0;
#pragma unroll
  for (int w = 0; w < THREADS / kWave; ++w)
    if (w < wave) base += tot[w];
  return base + incl - v;
}

// Wave 0: the digit whose bin holds the r-th largest key (bins taken in
// descending digit order) and the count of keys in the bins above it.
__device__ __forceinline__ void find_digit(const int* hist, int r, int* digit, int* above) {
  const int lane = threadIdx.x & (kWave - 1);
  // lane l: digits 255-4l, 254-4l, 253-4l, 252-4l = v.w, v.z, v.y, v.x
  const int4 v = *reinterpret_cast<const int4*>(hist + 252 - 4 * lane);
  const int s = v.x + v.y + v.z + v.w;
  const int incl = wave_incl_scan(s);
  const uint64_t hit = __ballot(incl >= r);
  const int first = hit ? __builtin_ctzll(hit) : kWave - 1;
  if (lane == first) {
    int ex = incl - s, d = 255 - 4 * lane;
    if (ex + v.w < r) {
      ex += v.w;
      --d;
      if (ex + v.z < r) {
        ex += v.z;
        --d;
        if (ex + v.y < r) {
          ex += v.y;
          --d;
        }
      }
    }
    *digit = d;
    *above = ex;
  }
}

// keys[0, cand) hold order keys of the candidates (written before a
// barrier); calls out(i, position) for every kept slot i in [0, budget),
// where budget = want + window.  All THREADS threads call it.  MAXPER > 0:
// every thread holds at most MAXPER candidates (cand <= THREADS * MAXPER),
// kept in registers; MAXPER = 0: any cand, read from LDS on every pass.
template <int THREADS, int MAXPER, typename OutFn>
__device__ __forceinline__ void block_select(const uint32_t* keys, int cand, int want, int window,
                                             SelectShared<THREADS>& sh, OutFn out) {
  const int tid = threadIdx.x, wave = tid / kWave;
  // each thread owns the contiguous positions [lo, hi); an odd run length
  // keeps the lanes of a wave on different LDS banks
  int per = (cand + THREADS - 1) / THREADS;
  if (MAXPER == 0) per |= 1;
  const int lo = min(tid * per, cand), hi = min(lo + per, cand);
  uint32_t kr[MAXPER > 0 ? MAXPER : 1];
  if (MAXPER > 0) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) kr[i] = lo + i < hi ? keys[lo + i] : 0u;
  }
  for (int b = tid; b < 512; b += THREADS) (&sh.hist[0][0])[b] = 0;
  lds_barrier();

  uint32_t prefix = 0u, mask = 0u;
  int r = want;   // keys still to take at or below the prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    int* h = sh.hist[pass & 1];
    if (MAXPER > 0) {
#pragma unroll
      for (int i = 0; i < MAXPER; ++i)
        if (lo + i < hi && (kr[i] & mask) == prefix) atomicAdd(&h[(kr[i] >> shift) & 255u], 1);
    } else {
      for (int j = tid; j < cand; j += THREADS) {
        const uint32_t kk = keys[j];
        if ((kk & mask) == prefix) atomicAdd(&h[(kk >> shift) & 255u], 1);
      }
    }
    lds_barrier();
    if (wave == 0) {
      find_digit(h, r, &sh.digit, &sh.above);
    } else {
      int* nxt = sh.hist[(pass + 1) & 1];
      for (int b = tid - kWave; b < 256; b += THREADS - kWave) nxt[b] = 0;
    }
    lds_barrier();
    prefix |= (uint32_t)sh.digit << shift;
    mask |= 0xFFu << shift;
    r -= sh.above;
  }
  // prefix = the want-th largest key; keep every larger key and the first r
  // equal ones in position order.  Counts below 2^16 pack into one scan.
  int cgt = 0, ceq = 0;
  if (MAXPER > 0) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i)
      if (lo + i < hi) {
        cgt += kr[i] > prefix;
        ceq += kr[i] == prefix;
      }
  } else {
    for (int j = lo; j < hi; ++j) {
      const uint32_t kk = keys[j];
      cgt += kk > prefix;
      ceq += kk == prefix;
    }
  }
  const int ex = block_excl_scan<THREADS>(cgt | (ceq << 16), sh.tot);
  const int gt_before = ex & 0xFFFF, eq_before = ex >> 16;
  int o = gt_before + min(eq_before, r);
  int eqi = eq_before;
  if (MAXPER > 0) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      if (lo + i < hi) {
        bool kp = kr[i] > prefix;
        if (kr[i] == prefix) kp = eqi++ < r;
        if (kp) out(o++, lo + i);
      }
    }
  } else {
    for (int j = lo; j < hi; ++j) {
      const uint32_t kk = keys[j];
      bool kp = kk > prefix;
      if (kk == prefix) kp = eqi++ < r;
      if (kp) out(o++, j);
    }
  }
  for (int i = tid; i < window; i += THREADS) out(want + i, cand + i);
}

}  // namespace rkv
