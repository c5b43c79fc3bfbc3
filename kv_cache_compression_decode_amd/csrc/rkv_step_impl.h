// The whole R-KV compression step of one unit in one workgroup, for units
// the single-pass scoring handles (bf16, up to UnitShape<D>::NMAX keys):
// score (rkv_unit_impl.h), select (rkv_select_impl.h), then compact -- the
// kept keys are still in registers from scoring, so K is read from HBM once
// and only written where a row moves; paged sequences report their freed
// blocks (R-KV project page on hysenlabs.com, "How R-KV decides what to
// drop": two-phase compaction, FREE_BLOCKS).  Outputs are the same as
// rkv_score + rkv_select + rkv_compact: the same score and selection code
// runs, and the compaction moves the same rows.
//
// Value rows: the last PRE rows of the unit are copied HBM -> LDS
// (global_load_lds, no registers) while the scoring arithmetic runs, issued
// in parts at its prefetch stages; the other moved value rows are read into
// registers after selection.  Every moved row is
// read before any is written, so the in-place move needs no ordering.
#pragma once

#include "rkv_select_impl.h"
#include "rkv_unit_impl.h"

namespace rkv {

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at lds + 16 l; lds must be the same for the whole wave.
__device__ __forceinline__ void load_to_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// LDS of the fused kernel besides the value-row buffer.
template <int D, int RT>
struct StepLds {
  static constexpr int NMAX = UnitShape<D>::NMAX;
  UnitLds<D, RT> unit;
  uint32_t keys[NMAX];           // score order keys, then destination slots
  int32_t keep[NMAX];
  SelectShared<kUnitThreads> sel;
  int first_moved;               // first slot that receives another row
  int lds_from;                  // first slot whose row comes from the LDS buffer
};

template <int D, int RT>
struct StepShape {
  static constexpr int ROWB = 2 * D;                        // bytes per bf16 row
  static constexpr int RPI = kWave * 16 / ROWB;             // rows per wave-wide 16-byte load
  static constexpr int GROUP = RPI * kUnitWaves;            // rows per workgroup-wide round
  static constexpr int kLdsBytes = 160 * 1024;              // LDS per workgroup on gfx950
  static constexpr int FREE = kLdsBytes - (int)sizeof(StepLds<D, RT>) - 512;
  static constexpr int PRE0 = FREE / ROWB / GROUP * GROUP;
  static constexpr int PRE = PRE0 < UnitShape<D>::NMAX ? PRE0 : UnitShape<D>::NMAX;
  static constexpr int ROUNDS = PRE / GROUP;
  static_assert(PRE >= GROUP, "value-row buffer must hold at least one round");
};

template <bool PAGED, int D, int RT>
__global__ __launch_bounds__(kUnitThreads) void step_unit_kernel(StepArgs sa) {
  using SS = StepShape<D, RT>;
  constexpr int NBW = UnitShape<D>::NBW;
  constexpr int NMAX = UnitShape<D>::NMAX;
  constexpr int KS = D / 32;
  constexpr int TPR = SS::ROWB / 16;              // threads per row (16 B each)
  constexpr int RPP = kUnitThreads / TPR;         // rows per pass
  const ScoreArgs& a = sa.s;
  __shared__ StepLds<D, RT> S;
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[SS::PRE * SS::ROWB];

  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  if (u.n == 0) return;   // past the device table's count
  if (sa.reset_status) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.status = 0u;   // nothing else of the call writes it
  } else if (step_aborted(a.status)) {
    return;   // the step failed a device check: leave everything untouched
  }
  const int n = u.n, budget = a.g.budget, window = a.g.window;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int pb = max(0, n - SS::PRE);             // rows [pb, n) go through vbuf
  const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(sa.v);

  KeyFrag<true, D> kf[NBW];
  unit_score<PAGED, D, RT>(
      a, u, S.unit, kf,
      [&](int stage) {
        KeyRows<PAGED> rows;
        rows.init(a.g, a.bt, u);
        // wave w, round i: rows RPI*(w + 16 i) .. +RPI-1 of the buffer, one
        // 16-byte piece per lane, landing at the wave's base + 16 * lane.
        // The rounds are spread over the prefetch stages -- except for the
        // paged layout, whose row addresses need block-table loads: waiting
        // for those would also wait for the rounds already in flight.
        constexpr int NST = PAGED ? 1 : kPrefetchStages;
        if (stage >= NST) return;
#pragma unroll
        for (int i = stage * SS::ROUNDS / NST; i < (stage + 1) * SS::ROUNDS / NST; ++i) {
          const int row0 = SS::RPI * (wave + kUnitWaves * i);
          const int pos = min(pb + row0 + lane / TPR, n - 1);
          load_to_lds16(vsrc + rows.at(pos) * 2 + (lane % TPR) * 16, vbuf + row0 * SS::ROWB);
        }
      },
      [&](int key, float sc) { S.keys[key] = order_key(sc); });
  if (t == 0) {
    S.first_moved = budget;
    S.lds_from = budget;
  }
  block_select_init(S.sel);
  lds_barrier();

  // The selection hands every token its destination slot (-1: evicted) in
  // dest, which takes over the order keys' LDS (they live in registers after
  // the selection's first barrier), and the keep list; meanwhile each thread
  // notes the first slot that moves and the first slot whose row is in vbuf
  // (keep is ascending).
  int32_t* krow = sa.keep + out_row(a.g, u) * budget;
  int* dest = reinterpret_cast<int*>(S.keys);
  int lo = budget, cut = budget;
  block_select<kUnitThreads, (NMAX + kUnitThreads - 1) / kUnitThreads>(
      S.keys, n - window, budget - window, window, S.sel,
      [&](int i, int pos) {
        S.keep[i] = pos;
        krow[i] = pos;
        dest[pos] = i;
        if (pos != i) lo = min(lo, i);
        if (pos >= pb) cut = min(cut, i);
      },
      [&](int pos) { dest[pos] = -1; });
  lo = (int)wave_minmax<false>((uint32_t)lo);   // slots are non-negative
  cut = (int)wave_minmax<false>((uint32_t)cut);
  if (lane == 0) {
    if (lo < budget) lds_min(&S.first_moved, lo);
    if (cut < budget) lds_min(&S.lds_from, cut);
  }
  lds_barrier();

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
  // V, moved slots [start, budget): [start, mid) from HBM through registers
  // (passes of RPP rows, at most 20 -- the key fragments are dead by now),
  // [mid, budget) from vbuf.  The register loads are unconditional (slots
  // clamped into [start, mid)) so that no branch makes a wave wait between
  // them; only slots below mid are stored from registers.  The value rows
  // are written with non-temporal stores (measured: faster than cached
  // stores here, while cached loads and key stores beat non-temporal ones).
  static_assert(NMAX <= 20 * RPP, "value rows must fit 20 register passes");
  const int piece = (t % TPR) * 16;
  uint8_t* vdst = reinterpret_cast<uint8_t*>(sa.v) + piece;
  const uint8_t* vget = vsrc + piece;
  const int rr = t / TPR;
  const int start = S.first_moved;
  const int mid = max(start, S.lds_from);
  const int last = max(mid - 1, 0);
#define RKV_VLOAD(r)                     \
  const int s##r = start + r * RPP + rr; \
  const uint4 b##r = *reinterpret_cast<const uint4*>(vget + rows.at(S.keep[min(s##r, last)]) * 2);
#define RKV_VSTORE(r) \
  if (s##r < mid) stream_store(reinterpret_cast<uint4*>(vdst + rows.at(s##r) * 2), b##r);
  RKV_VLOAD(0) RKV_VLOAD(1) RKV_VLOAD(2) RKV_VLOAD(3) RKV_VLOAD(4)
  RKV_VLOAD(5) RKV_VLOAD(6) RKV_VLOAD(7) RKV_VLOAD(8) RKV_VLOAD(9)
  RKV_VLOAD(10) RKV_VLOAD(11) RKV_VLOAD(12) RKV_VLOAD(13) RKV_VLOAD(14)
  RKV_VLOAD(15) RKV_VLOAD(16) RKV_VLOAD(17) RKV_VLOAD(18) RKV_VLOAD(19)
  __builtin_amdgcn_s_waitcnt(0);   // also completes this wave's vbuf loads
  __syncthreads();
  RKV_VSTORE(0) RKV_VSTORE(1) RKV_VSTORE(2) RKV_VSTORE(3) RKV_VSTORE(4)
  RKV_VSTORE(5) RKV_VSTORE(6) RKV_VSTORE(7) RKV_VSTORE(8) RKV_VSTORE(9)
  RKV_VSTORE(10) RKV_VSTORE(11) RKV_VSTORE(12) RKV_VSTORE(13) RKV_VSTORE(14)
  RKV_VSTORE(15) RKV_VSTORE(16) RKV_VSTORE(17) RKV_VSTORE(18) RKV_VSTORE(19)
#undef RKV_VLOAD
#undef RKV_VSTORE
  for (int s = mid + rr; s < budget; s += RPP) {
    const uint4 v = *reinterpret_cast<const uint4*>(vbuf + (S.keep[s] - pb) * SS::ROWB + piece);
    stream_store(reinterpret_cast<uint4*>(vdst + rows.at(s) * 2), v);
  }

  if (PAGED && sa.free_blocks != nullptr && u.l == 0 && u.h == 0) {
    const int bs = 1 << a.g.bs_shift;
    const int first = (budget + bs - 1) / bs, last_blk = (n + bs - 1) / bs;
    int32_t* out = sa.free_blocks + free_off(a.g, a.tt, u.ti);
    for (int b = first + t; b < last_blk; b += kUnitThreads)
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
