// Scoring of units longer than one workgroup's registers hold (bf16, more
// than UnitShape<D>::NMAX keys), reading every key from HBM once.  Same
// quantities as the single-pass kernel (R-KV project page on hysenlabs.com,
// "How R-KV decides what to drop"; hotdry blog post, R-KV section).
//
// A unit is split into C contiguous key spans, one per workgroup, each held
// in registers like a whole unit in score_unit_kernel.  The span's row
// statistics (max and sum of exp2) and direction sum are published in the
// workspace; once all C spans of the unit have published, every span merges
// the C records in span order (so the C workgroups compute identical unit
// statistics) and finishes its own keys' importance, redundancy and score.
//
// Units are launched P at a time (P * C workgroups: as many as are resident
// on the device at once), unit unit0 + i taken by workgroups C*i .. C*i+C-1,
// so the C workgroups a span waits for are all running.  Work of other kinds
// on other streams can only delay some of them (it finishes and frees its
// room); two such span launches at once on one device could hold each
// other's room, which is why the interface asks for them on one stream.  The wait is a
// spin on a per-unit counter (zeroed by a small kernel first), bounded at
// one second so that no launch can hang the device; a launch that reached
// the bound would finish with wrong scores -- it is never reached when the
// launch's workgroups are dispatched.
#pragma once

#include <algorithm>
#include <atomic>

#include "rkv_unit_impl.h"

namespace rkv {

struct LongArgs {
  int32_t chunks;       // C: workgroups (key spans) per unit
  int32_t wait_ticks;   // bound on the wait for the other spans (s_memrealtime, 100 MHz)
  int32_t unit0;        // first unit of this launch: workgroup w takes span w % C of unit0 + w / C
};

// Counter of unit ui: the first word of record slot C of the unit (the
// workspace holds max_chunks > C record slots per unit).
__device__ __forceinline__ uint32_t* long_counter(const ScoreArgs& a, int ui, int C) {
  return reinterpret_cast<uint32_t*>(a.part + ((size_t)ui * a.max_chunks + C) * a.rec);
}

static __global__ void long_zero_kernel(ScoreArgs a, int C, int units) {
  const int ui = blockIdx.x * blockDim.x + threadIdx.x;
  if (ui < units) *long_counter(a, ui, C) = 0u;
}

// Every thread's earlier global stores are published, then this workgroup
// adds one to the unit's counter and waits until it reaches target (or the
// time bound passes).  All threads call it.
__device__ __forceinline__ void span_signal_wait(uint32_t* cnt, uint32_t target, int wait_ticks) {
  __syncthreads();   // every store of the workgroup performed
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target &&
           __builtin_amdgcn_s_memrealtime() - t_start < (uint64_t)wait_ticks)
      __builtin_amdgcn_s_sleep(2);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// The span's record (row max, raw sum, direction sum) into slot c of the
// unit's records; identity values for a span without keys.
template <int D, int RT>
__device__ __forceinline__ void publish_span_stats(UnitLds<D, RT>& L, float* recs, int rec, int c,
                                                   int gw, bool empty) {
  __syncthreads();   // the span's statistics are in LDS
  const int t = threadIdx.x;
  float* mine = recs + (size_t)c * rec;
  if (t < gw) {
    mine[t] = empty ? -INFINITY : L.row_m[t];
    mine[gw + t] = empty ? 0.f : L.row_iz[t];
  }
  if (t < D) mine[2 * gw + t] = empty ? 0.f : L.red_s[t][0];
}

// The unit's row statistics and direction-sum rows from the C records,
// merged in span order (every span computes the same values).
template <int D, int RT>
__device__ __forceinline__ void merge_span_stats(UnitLds<D, RT>& L, const float* recs, int rec, int C,
                                                 int gw) {
  constexpr int QP = UnitLds<D, RT>::QP;
  const int t = threadIdx.x;
  if (t < RT * 16) {
    float mm = -INFINITY, zz = 0.f;
    if (t < gw)
      for (int cc = 0; cc < C; ++cc)
        merge_stats(mm, zz, recs[(size_t)cc * rec + t], recs[(size_t)cc * rec + gw + t]);
    L.row_m[t] = t < gw ? mm : INFINITY;   // log2 units; other rows add nothing
    L.row_iz[t] = t < gw ? 1.f / (zz * (float)gw) : 0.f;
  }
  if (t < D) {   // the unit's sum of khat, split into the two bf16 rows gw and gw + 1
    float sv = 0.f;
    for (int cc = 0; cc < C; ++cc) sv += recs[(size_t)cc * rec + 2 * gw + t];
    const uint32_t hi = f2bf_bits(sv);
    L.q[gw * QP + t] = (uint16_t)hi;
    L.q[(gw + 1) * QP + t] = (uint16_t)f2bf_bits(sv - __uint_as_float(hi << 16));
  }
}

template <bool PAGED, int D, int RT>
__global__ __launch_bounds__(kUnitThreads) void score_long_kernel(ScoreArgs a, LongArgs la) {
  __shared__ UnitLds<D, RT> L;
  KeyFrag<true, D> kf[UnitShape<D>::NBW];
  const int C = la.chunks;
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  const int c = blockIdx.x % C, t = threadIdx.x, gw = a.gw;
  {
    const int ui = la.unit0 + blockIdx.x / C;
    if (ui >= units) return;
    const Unit u = decode_unit(a.g, a.tt, ui);
    if (u.n == 0) return;   // past the device table's count: all C workgroups skip it
    const int k0 = (int)((int64_t)c * u.n / C), k1 = (int)((int64_t)(c + 1) * u.n / C);
    float* recs = a.part + (size_t)ui * a.max_chunks * a.rec;
    uint32_t* cnt = long_counter(a, ui, C);

    // publish this span's record, wait for the unit's other spans, merge
    auto exchange = [&](bool empty) {
      publish_span_stats(L, recs, a.rec, c, gw, empty);
      span_signal_wait(cnt, (uint32_t)C, la.wait_ticks);
      if (!empty) merge_span_stats(L, recs, a.rec, C, gw);
    };

    if (k1 > k0)
      unit_score_span<PAGED, D, RT, true>(a, u, k0, k1 - k0, L, kf, [](int) {}, [](int, float) {},
                                          [&] { exchange(false); });
    else
      exchange(true);   // a unit shorter than C: this span holds no key
  }
}

template <bool PAGED, int D, int RT>
hipError_t launch_long_t(const ScoreArgs& a, int chunks, hipStream_t st) {
  // resident workgroups: per device, computed once (atomic: calls may come
  // from several host threads; a repeated computation stores the same value)
  static std::atomic<int> grid_of[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int resident = grid_of[dev].load(std::memory_order_relaxed);
  if (resident == 0) {
    int cus = 0, occ = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
             &occ, reinterpret_cast<const void*>(score_long_kernel<PAGED, D, RT>), kUnitThreads, 0)) !=
        hipSuccess)
      return e;
    if (cus <= 0 || occ <= 0) return hipErrorInvalidConfiguration;
    resident = cus * occ;
    grid_of[dev].store(resident, std::memory_order_relaxed);
  }
  const int per = resident / chunks;   // units whose spans are all resident at once
  if (per < 1) return hipErrorInvalidConfiguration;
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  hipLaunchKernelGGL(long_zero_kernel, dim3((units + 255) / 256), dim3(256), 0, st, a, chunks, units);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int u0 = 0; u0 < units; u0 += per) {
    LongArgs la{chunks, 100000000, u0};   // 1 s: far beyond any wait of a resident launch
    const int grid = std::min(per, units - u0) * chunks;
    hipLaunchKernelGGL((score_long_kernel<PAGED, D, RT>), dim3(grid), dim3(kUnitThreads), 0, st, a, la);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool PAGED, int D>
hipError_t dispatch_long(const ScoreArgs& a, int chunks, int rt2, hipStream_t st) {
  typedef hipError_t (*Fn)(const ScoreArgs&, int, hipStream_t);
  static const Fn fns[kUnitMaxRowTiles] = {launch_long_t<PAGED, D, 1>, launch_long_t<PAGED, D, 2>,
                                           launch_long_t<PAGED, D, 3>, launch_long_t<PAGED, D, 4>,
                                           launch_long_t<PAGED, D, 5>};
  return fns[rt2 - 1](a, chunks, st);
}

}  // namespace rkv
