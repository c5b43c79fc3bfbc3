// Workgroup-wide selection over scores staged in LDS, shared by the select
// kernel and the fused step kernel.  Per unit: keep the last `window`
// tokens and the budget - window highest-scoring others (hotdry blog post,
// R-KV section: keep what is important and not redundant; R-KV project page,
// "How R-KV decides what to drop": budget and local window); equal scores
// keep the lower position; output in ascending position.
//
// Scores are mapped to order-preserving uint32 keys; an MSB-first radix
// select finds the (budget - window)-th largest key t and how many keys equal
// to t are kept; one workgroup scan then gives every thread the output
// offset of its contiguous run of positions.  The digits start below the
// bits that every key of the unit shares (from the keys' min and max), and
// the passes stop once the bin holding t is taken whole, so a unit's scores,
// which share their leading bits, usually need two or three 8-bit passes.
// Each pass has its own histogram (all cleared up front) and costs one
// barrier: after it every wave reads the histogram and finds the digit
// itself.  A wave adds its lanes' most common digit with one atomic (ballot)
// before the remaining lanes add their own.
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
  __attribute__((aligned(16))) int hist[4][256];
  int tot[THREADS / kWave];
  uint32_t kmin, kmax;
};

// Clears the histograms and the min / max; all threads call it, and a
// barrier must separate it from block_select.
template <int THREADS>
__device__ __forceinline__ void block_select_init(SelectShared<THREADS>& sh) {
  for (int b = threadIdx.x; b < 4 * 256; b += THREADS) (&sh.hist[0][0])[b] = 0;
  if (threadIdx.x == 0) {
    sh.kmin = ~0u;
    sh.kmax = 0u;
  }
}

// Min / max over the 64 lanes of a wave (DPP within rows of 16, then the
// lane swaps across rows); every lane gets the result.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return MAX ? max(x, y) : min(x, y); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));   // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));   // row_mirror
  auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(p[0], p[1]);
  p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(p[0], p[1]);
}

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

// Every wave: the digit whose bin holds the r-th largest key (bins taken in
// descending digit order), the count of keys in the bins above it and the
// count in its own bin (wave-uniform results).
__device__ __forceinline__ void find_digit(const int* hist, int r, int& digit, int& above,
                                           int& count) {
  const int lane = threadIdx.x & (kWave - 1);
  // lane l: digits 255-4l, 254-4l, 253-4l, 252-4l = v.w, v.z, v.y, v.x
  const int4 v = *reinterpret_cast<const int4*>(hist + 252 - 4 * lane);
  const int s = v.x + v.y + v.z + v.w;
  const int incl = wave_incl_scan(s);
  const uint64_t hit = __ballot(incl >= r);
  const int first = hit ? __builtin_ctzll(hit) : kWave - 1;
  int ex = incl - s, d = 255 - 4 * lane, c = v.w;
  if (ex + v.w < r) {
    ex += v.w;
    --d;
    c = v.z;
    if (ex + v.z < r) {
      ex += v.z;
      --d;
      c = v.y;
      if (ex + v.y < r) {
        ex += v.y;
        --d;
        c = v.x;
      }
    }
  }
  digit = __builtin_amdgcn_readlane(d, first);
  above = __builtin_amdgcn_readlane(ex, first);
  count = __builtin_amdgcn_readlane(c, first);
}

// hist[dg] += 1 for every lane with on set.  All lanes of the wave call it.
// The digit of the first such lane is counted for the whole wave with one
// atomic (in a unit's first pass most lanes share it); the lanes left over
// add 1 each.
__device__ __forceinline__ void hist_add(int* hist, int dg, bool on) {
  constexpr int kPeel = 1;
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t todo = __ballot(on);
#pragma unroll
  for (int it = 0; it < kPeel; ++it) {
    if (todo == 0) break;
    const int leader = __builtin_ctzll(todo);
    const int dl = __builtin_amdgcn_readlane(dg, leader);
    const bool m = on && dg == dl;
    const uint64_t same = __ballot(m);
    if (lane == leader) lds_add(&hist[dl], __popcll(same));
    todo &= ~same;
    on = on && !m;
  }
  if (on) lds_add(&hist[dg], 1);
}

// keys[0, cand) hold order keys of the candidates (written before a
// barrier that also follows block_select_init); calls out(i, position) for
// every kept slot i in [0, budget), where budget = want + window, and
// drop(position) for every candidate not kept.  All THREADS threads call it.
// MAXPER > 0: every thread holds at most MAXPER candidates (cand <= THREADS *
// MAXPER), kept in registers, and keys[] is not read after the first barrier
// (the caller may reuse it from the callbacks on); MAXPER = 0: any cand, read
// from LDS on every pass.
template <int THREADS, int MAXPER, typename OutFn, typename DropFn>
__device__ __forceinline__ void block_select(const uint32_t* keys, int cand, int want, int window,
                                             SelectShared<THREADS>& sh, OutFn out, DropFn drop) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // each thread owns the contiguous positions [lo, hi); an odd run length
  // keeps the lanes of a wave on different LDS banks
  int per = (cand + THREADS - 1) / THREADS;
  if (MAXPER == 0) per |= 1;
  const int lo = min(tid * per, cand), hi = min(lo + per, cand);
  uint32_t kr[MAXPER > 0 ? MAXPER : 1];
  uint32_t kmin = ~0u, kmax = 0u;
  if (MAXPER > 0) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      kr[i] = lo + i < hi ? keys[lo + i] : 0u;
      if (lo + i < hi) {
        kmin = min(kmin, kr[i]);
        kmax = max(kmax, kr[i]);
      }
    }
  } else {
    for (int j = lo; j < hi; ++j) {
      kmin = min(kmin, keys[j]);
      kmax = max(kmax, keys[j]);
    }
  }
  kmin = wave_minmax<false>(kmin);
  kmax = wave_minmax<true>(kmax);
  if (lane == 0) {
    lds_min(&sh.kmin, kmin);
    lds_max(&sh.kmax, kmax);
  }
  lds_barrier();

  // bits [low, 32) of every key equal those of the min: start below them
  const uint32_t diff = sh.kmin ^ sh.kmax;
  int low = diff ? 32 - __builtin_clz(diff) : 0;
  uint32_t mask = low < 32 ? ~((1u << low) - 1u) : 0u;
  uint32_t prefix = sh.kmin & mask;
  int r = want;   // keys still to take among those matching prefix under mask
#pragma unroll   // a constant histogram address per pass keeps its LDS accesses
                 // distinguishable from the value-row stream
  for (int pass = 0; pass < 4; ++pass) {
    if (low == 0) break;
    const int shift = max(low - 8, 0);
    const uint32_t dmask = (1u << (low - shift)) - 1u;
    int* h = sh.hist[pass];
    if (MAXPER > 0) {
#pragma unroll
      for (int i = 0; i < MAXPER; ++i)
        hist_add(h, (kr[i] >> shift) & dmask, lo + i < hi && (kr[i] & mask) == prefix);
    } else {
      // wave-uniform trip count: every lane takes part in the ballots
      for (int j0 = tid - lane; j0 < cand; j0 += THREADS) {
        const int j = j0 + lane;
        const uint32_t kk = keys[min(j, cand - 1)];
        hist_add(h, (kk >> shift) & dmask, j < cand && (kk & mask) == prefix);
      }
    }
    lds_barrier();
    int digit, above, count;
    find_digit(h, r, digit, above, count);
    prefix |= (uint32_t)digit << shift;
    mask |= dmask << shift;
    r -= above;
    low = shift;
    if (count == r) break;   // the whole bin is kept: its order does not matter
  }
  // keep every key above prefix (under mask) and the first r equal ones in
  // position order.  Counts below 2^16 pack into one scan.
  int cgt = 0, ceq = 0;
  if (MAXPER > 0) {
#pragma unroll
    for (int i = 0; i < MAXPER; ++i)
      if (lo + i < hi) {
        cgt += (kr[i] & mask) > prefix;
        ceq += (kr[i] & mask) == prefix;
      }
  } else {
    for (int j = lo; j < hi; ++j) {
      const uint32_t kk = keys[j] & mask;
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
        const uint32_t kk = kr[i] & mask;
        bool kp = kk > prefix;
        if (kk == prefix) kp = eqi++ < r;
        if (kp)
          out(o++, lo + i);
        else
          drop(lo + i);
      }
    }
  } else {
    for (int j = lo; j < hi; ++j) {
      const uint32_t kk = keys[j] & mask;
      bool kp = kk > prefix;
      if (kk == prefix) kp = eqi++ < r;
      if (kp)
        out(o++, j);
      else
        drop(j);
    }
  }
  for (int i = tid; i < window; i += THREADS) out(want + i, cand + i);
}

}  // namespace rkv
