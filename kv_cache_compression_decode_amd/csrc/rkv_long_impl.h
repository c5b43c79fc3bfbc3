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
// One launch takes every unit.  A workgroup's span is given by a ticket it
// draws when it starts (an atomic counter): consecutive tickets are the
// spans of one unit, in unit order.  A span therefore only waits for spans that
// started before it or that the next starting workgroups will take: while
// a unit's spans are not all running, every other running workgroup belongs
// to a unit whose spans all are, so it finishes and frees room for the next
// ticket (this needs room for a unit's workgroups on the device, which the
// launch checks).  Units start one after another as room frees.  Work of
// other kinds on other streams can only delay some of them (it finishes and
// frees its room); two such span launches at once on one device could hold
// each other's room, which is why the interface asks for them on one
// stream.  The wait is a spin on a per-unit counter (zeroed, with the ticket
// counter, by a small kernel first), bounded (one second unless the caller
// sets another bound) so that no launch can hang the device; it is never
// reached when the launch's workgroups are dispatched.  A span whose wait
// reaches the bound sets kSpanTimeout in the call's status word and
// finishes with wrong scores; the selection and compaction kernels of the
// call then leave the keep rows and the cache untouched.
#pragma once

#include <algorithm>
#include <atomic>

#include "rkv_unit_impl.h"

namespace rkv {

struct LongArgs {
  int64_t wait_ticks;   // bound on the wait for the other spans (s_memrealtime, 100 MHz)
  int32_t chunks;       // C: workgroups (key spans) per unit
};

// Counter of unit ui: the first word of record slot C of the unit (the
// workspace holds max_chunks > C record slots per unit).
__device__ __forceinline__ uint32_t* long_counter(const ScoreArgs& a, int ui, int C) {
  return reinterpret_cast<uint32_t*>(a.part + ((size_t)ui * a.max_chunks + C) * a.rec);
}

// Ticket counter of a launch: word 32 of unit 0's counter slot (a record
// slot holds 2 G w + D >= 66 words), on its own 128-byte line.
__device__ __forceinline__ uint32_t* long_tickets(const ScoreArgs& a, int C) {
  return long_counter(a, 0, C) + 32;
}

static __global__ void long_zero_kernel(ScoreArgs a, int C, int units) {
  const int ui = blockIdx.x * blockDim.x + threadIdx.x;
  if (ui < units) *long_counter(a, ui, C) = 0u;
  if (ui == 0) *long_tickets(a, C) = 0u;
  if (a.reset_status) clear_status_first(a.status);
}

// The workgroup's record stores (agent-scope atomic stores: written through
// to the device's coherence point) have completed, then this workgroup adds
// one to the unit's counter and waits until it reaches target (or the time
// bound passes: then kSpanTimeout goes into the status word; a bound of 0
// gives up at once and always reports it).  All threads call it.  The
// records are read back with agent-scope atomic loads, so neither side
// writes back or invalidates the XCD's L2 (an agent-scope fence would do
// both, for every span).
__device__ __forceinline__ void span_signal_wait(uint32_t* cnt, uint32_t target, int64_t wait_ticks,
                                                 uint32_t* status) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's record stores are done
  __syncthreads();                                    // ... and every other thread's
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    bool done = false;
    if (wait_ticks > 0) {
      for (;;) {
        done = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target;
        if (done || __builtin_amdgcn_s_memrealtime() - t_start >= (uint64_t)wait_ticks) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (!done && status != nullptr)
      __hip_atomic_fetch_or(status, kSpanTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

__device__ __forceinline__ void rec_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rec_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    rec_store(mine + t, empty ? -INFINITY : L.row_m[t]);
    rec_store(mine + gw + t, empty ? 0.f : L.row_iz[t]);
  }
  if (t < D) rec_store(mine + 2 * gw + t, empty ? 0.f : L.red_s[t][0]);
}

// The unit's row statistics and direction-sum rows from the C records,
// merged in span order (every span computes the same values).  The records
// are read kRecBatch spans at a time, each batch's loads issued together:
// they come from the coherence point, so one at a time would pay its
// latency C times.
constexpr int kRecBatch = 4;

template <int D, int RT>
__device__ __forceinline__ void merge_span_stats(UnitLds<D, RT>& L, const float* recs, int rec, int C,
                                                 int gw) {
  constexpr int QP = UnitLds<D, RT>::QP;
  const int t = threadIdx.x;
  if (t < RT * 16) {
    float mm = -INFINITY, zz = 0.f;
    if (t < gw)
      for (int c0 = 0; c0 < C; c0 += kRecBatch) {
        float m4[kRecBatch], z4[kRecBatch];
#pragma unroll
        for (int i = 0; i < kRecBatch; ++i) {
          const size_t cc = (size_t)min(c0 + i, C - 1);
          m4[i] = rec_load(recs + cc * rec + t);
          z4[i] = rec_load(recs + cc * rec + gw + t);
        }
#pragma unroll
        for (int i = 0; i < kRecBatch; ++i)
          if (c0 + i < C) merge_stats(mm, zz, m4[i], z4[i]);
      }
    L.row_m[t] = t < gw ? mm : INFINITY;   // log2 units; other rows add nothing
    L.row_iz[t] = t < gw ? 1.f / (zz * (float)gw) : 0.f;
  }
  if (t < D) {   // the unit's sum of khat, split into the two bf16 rows gw and gw + 1
    float sv = 0.f;
    for (int c0 = 0; c0 < C; c0 += kRecBatch) {
      float s4[kRecBatch];
#pragma unroll
      for (int i = 0; i < kRecBatch; ++i)
        s4[i] = rec_load(recs + (size_t)min(c0 + i, C - 1) * rec + 2 * gw + t);
#pragma unroll
      for (int i = 0; i < kRecBatch; ++i)
        if (c0 + i < C) sv += s4[i];
    }
    const uint32_t hi = f2bf_bits(sv);
    L.q[gw * QP + t] = (uint16_t)hi;
    L.q[(gw + 1) * QP + t] = (uint16_t)f2bf_bits(sv - __uint_as_float(hi << 16));
  }
}

template <bool PAGED, int D, int RT>
__global__ __launch_bounds__(kUnitThreads) void score_long_kernel(ScoreArgs a, LongArgs la) {
  __shared__ UnitLds<D, RT> L;
  __shared__ uint32_t ticket;
  KeyFrag<true, D> kf[UnitShape<D>::NBW];
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  const int t = threadIdx.x, gw = a.gw;
  // a bad block id (set before this launch, so every span reads the same
  // value): the pool must not be read
  if (a.check_blocks && step_aborted(a.status, kBadBlockId)) return;
  const int C = la.chunks;
  if (t == 0) ticket = __hip_atomic_fetch_add(long_tickets(a, C), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int c = (int)(ticket % (uint32_t)C);
  {
    const int ui = (int)(ticket / (uint32_t)C);
    if (ui >= units) return;
    const Unit u = decode_unit(a.g, a.tt, ui);
    if (u.n == 0) return;   // past the device table's count: all C workgroups skip it
    const int k0 = (int)((int64_t)c * u.n / C), k1 = (int)((int64_t)(c + 1) * u.n / C);
    float* recs = a.part + (size_t)ui * a.max_chunks * a.rec;
    uint32_t* cnt = long_counter(a, ui, C);

    // publish this span's record, wait for the unit's other spans, merge
    auto exchange = [&](bool empty) {
      publish_span_stats(L, recs, a.rec, c, gw, empty);
      span_signal_wait(cnt, (uint32_t)C, la.wait_ticks, a.status);
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
  if (resident < chunks) return hipErrorInvalidConfiguration;   // a unit's spans must fit at once
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  hipLaunchKernelGGL(long_zero_kernel, dim3((units + 255) / 256), dim3(256), 0, st, a, chunks, units);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  LongArgs la{span_wait_ticks(), chunks};   // default 1 s: far beyond any wait of a dispatched span
  hipLaunchKernelGGL((score_long_kernel<PAGED, D, RT>), dim3(units * chunks), dim3(kUnitThreads), 0, st, a,
                     la);
  return hipGetLastError();
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
