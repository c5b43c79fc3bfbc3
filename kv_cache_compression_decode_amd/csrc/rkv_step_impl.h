// The whole R-KV compression step of one unit in one workgroup, for units
// the single-pass scoring handles (bf16, up to UnitShape<D>::NMAX keys):
// score (rkv_unit_impl.h), select (rkv_select_impl.h), then compact -- the
// kept keys are still in registers from scoring, so K is read from HBM once
// and only written where a row moves; all moved V rows are read into
// registers before any is written;
// paged sequences report their freed blocks (R-KV project page on
// hysenlabs.com, "How R-KV decides what to drop": two-phase compaction,
// FREE_BLOCKS).  Outputs are the same as rkv_score + rkv_select +
// rkv_compact: the same score and selection code runs, and the compaction
// moves the same rows.
#pragma once

#include "rkv_select_impl.h"
#include "rkv_unit_impl.h"

namespace rkv {


template <bool PAGED, int D, int RT>
__global__ __launch_bounds__(kUnitThreads) void step_unit_kernel(StepArgs sa) {
  constexpr int NBW = UnitShape<D>::NBW;
  constexpr int NMAX = UnitShape<D>::NMAX;
  constexpr int KS = D / 32;
  constexpr int TPR = D * 2 / 16;                 // threads per bf16 row (16 B each)
  constexpr int RPP = kUnitThreads / TPR;         // rows per pass
  const ScoreArgs& a = sa.s;
  __shared__ UnitLds<D, RT> L;
  __shared__ uint32_t keys_s[NMAX];               // score order keys, then destination slots
  __shared__ int32_t keep_s[NMAX];
  __shared__ SelectShared<kUnitThreads> ssh;
  __shared__ int first_moved;

  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  const int n = u.n, budget = a.g.budget, window = a.g.window;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, g4 = lane >> 4;

  KeyFrag<true, D> kf[NBW];
  unit_score<PAGED, D, RT>(a, u, L, kf, [&](int key, float sc) { keys_s[key] = order_key(sc); });
  if (t == 0) first_moved = budget;
  __syncthreads();

  int32_t* krow = sa.keep + out_row(a.g, u) * budget;
  block_select<kUnitThreads, (NMAX + kUnitThreads - 1) / kUnitThreads>(
      keys_s, n - window, budget - window, window, ssh, [&](int i, int pos) {
        keep_s[i] = pos;
        krow[i] = pos;
      });
  __syncthreads();
  // destination slot of every token (-1: evicted); first slot that moves
  int* dest = reinterpret_cast<int*>(keys_s);
  for (int j = t; j < n; j += kUnitThreads) dest[j] = -1;
  __syncthreads();
  int lo = budget;
  for (int i = t; i < budget; i += kUnitThreads) {
    const int p = keep_s[i];
    dest[p] = i;
    if (p != i) lo = min(lo, i);
  }
  if (lo < budget) atomicMin(&first_moved, lo);
  __syncthreads();

  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
  // K: every kept row is in registers (all reads are done); write moved rows
  uint16_t* kbase = reinterpret_cast<uint16_t*>(sa.k);
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
    if (key < n) {
      const int slot = dest[key];
      if (slot >= 0 && slot != key) {
        uint16_t* p = kbase + rows.at(slot) + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<uint4*>(p + 32 * ks) = kf[j].w[ks];
      }
    }
  }
  // V: every moved row (slots first_moved .. budget-1, at most NMAX / RPP
  // passes of RPP rows) is read into registers -- freed by the key fragments
  // -- before any is written, so the in-place move needs no ordering.
  static_assert(NMAX <= 20 * RPP, "value rows must fit 20 register passes");
  uint8_t* vbase = reinterpret_cast<uint8_t*>(sa.v) + (t % TPR) * 16;
  const int rr = t / TPR;
  const int start = first_moved;
#define RKV_VLOAD(r)                                                                     \
  const int s##r = start + r * RPP + rr;                                                 \
  uint4 b##r = make_uint4(0, 0, 0, 0);                                                   \
  if (s##r < budget) b##r = *reinterpret_cast<const uint4*>(vbase + rows.at(keep_s[s##r]) * 2);
#define RKV_VSTORE(r) \
  if (s##r < budget) *reinterpret_cast<uint4*>(vbase + rows.at(s##r) * 2) = b##r;
  RKV_VLOAD(0) RKV_VLOAD(1) RKV_VLOAD(2) RKV_VLOAD(3) RKV_VLOAD(4)
  RKV_VLOAD(5) RKV_VLOAD(6) RKV_VLOAD(7) RKV_VLOAD(8) RKV_VLOAD(9)
  RKV_VLOAD(10) RKV_VLOAD(11) RKV_VLOAD(12) RKV_VLOAD(13) RKV_VLOAD(14)
  RKV_VLOAD(15) RKV_VLOAD(16) RKV_VLOAD(17) RKV_VLOAD(18) RKV_VLOAD(19)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  RKV_VSTORE(0) RKV_VSTORE(1) RKV_VSTORE(2) RKV_VSTORE(3) RKV_VSTORE(4)
  RKV_VSTORE(5) RKV_VSTORE(6) RKV_VSTORE(7) RKV_VSTORE(8) RKV_VSTORE(9)
  RKV_VSTORE(10) RKV_VSTORE(11) RKV_VSTORE(12) RKV_VSTORE(13) RKV_VSTORE(14)
  RKV_VSTORE(15) RKV_VSTORE(16) RKV_VSTORE(17) RKV_VSTORE(18) RKV_VSTORE(19)
#undef RKV_VLOAD
#undef RKV_VSTORE

  if (PAGED && sa.free_blocks != nullptr && u.l == 0 && u.h == 0) {
    const int bs = 1 << a.g.bs_shift;
    const int first = (budget + bs - 1) / bs, last = (n + bs - 1) / bs;
    int32_t* out = sa.free_blocks + a.tt.free_off[u.ti];
    for (int b = first + t; b < last; b += kUnitThreads)
      out[b - first] = a.bt[(int64_t)u.s * a.g.maxblk + b];
  }
}

template <bool PAGED, int D, int RT>
hipError_t launch_step_t(const StepArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((step_unit_kernel<PAGED, D, RT>), dim3(units), dim3(kUnitThreads), 0, st, a);
  return hipGetLastError();
}

template <bool PAGED, int D>
hipError_t dispatch_step(const StepArgs& a, int units, int rt2, hipStream_t st) {
  typedef hipError_t (*Fn)(const StepArgs&, int, hipStream_t);
  static const Fn fns[kUnitMaxRowTiles] = {launch_step_t<PAGED, D, 1>, launch_step_t<PAGED, D, 2>,
                                           launch_step_t<PAGED, D, 3>, launch_step_t<PAGED, D, 4>,
                                           launch_step_t<PAGED, D, 5>};
  return fns[rt2 - 1](a, units, st);
}

}  // namespace rkv
