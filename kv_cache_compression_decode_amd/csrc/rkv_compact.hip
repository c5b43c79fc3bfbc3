// Compaction of the R-KV compression step: for each triggered unit, slot i of
// K and of V receives the row of token keep[i], in place, and the paged
// layout reports the blocks the sequence no longer uses (R-KV project page
// on hysenlabs.com, section "How R-KV decides what to drop": two-phase
// compaction, FREE_BLOCKS back to the allocator).
//
// In place without a second buffer: keep is ascending with keep[i] >= i, so
// the row written at slot i is read only by slots <= i.  A workgroup walks
// its unit's slots in tiles of ascending order; each tile is read into
// registers (phase 1), the workgroup waits for every read, then writes
// (phase 2).  Reads of tile t+1 touch rows >= its first slot, which no
// earlier tile writes, so they are issued before the writes of tile t and
// both are in flight together.  The keep row is staged in LDS first, and
// the walk starts at the first slot that moves (keep[i] == i below it).
//
// One 1024-thread workgroup per (unit, K or V); each row is read by
// consecutive lanes, 16 bytes per lane.  (Splitting the rows into column
// parts over more workgroups measured slower: whole rows per workgroup give
// the longest contiguous accesses; 1024 threads keep 128 KB of rows in
// flight per workgroup, which the batches of few units need.)
#include "rkv_device.h"
#include "rkv_launch.h"

namespace rkv {

namespace {
constexpr int kCompactRows = 8;        // rows per thread per tile (named registers below)
constexpr int kCompactThreads = 1024;  // per workgroup: 64 rows of 256 bytes per pass

// Element offset of token t's row; base = head_base of the unit.
template <bool PAGED>
__device__ __forceinline__ int64_t row_at(const CompactArgs& a, const Unit& u, int64_t base, int t) {
  if constexpr (PAGED) {
    const int blk = a.bt[(int64_t)u.s * a.g.maxblk + (t >> a.g.bs_shift)];
    const int64_t blk_stride = ((int64_t)a.g.hkv << a.g.bs_shift) * a.g.d;
    return base + blk * blk_stride + (int64_t)(t & ((1 << a.g.bs_shift) - 1)) * a.g.d;
  } else {
    return base + (int64_t)t * a.g.d;
  }
}

}  // namespace

// TPR: threads per row (row bytes / 16)
template <bool PAGED, int TPR>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactArgs a) {
  constexpr int NT = kCompactThreads, R = kCompactRows;
  constexpr int RPP = NT / TPR;         // rows per pass
  constexpr int TILE = RPP * R;         // rows per read/write round
  extern __shared__ int32_t keep_s[];
  __shared__ int first_moved;

  const int which = blockIdx.x & 1;
  const int unit_id = blockIdx.x / 2;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  if (u.n == 0) return;   // past the device table's count
  if (step_aborted(a.status)) return;   // the step failed a device check: cache untouched
  const int tid = threadIdx.x;
  const int64_t hb = head_base(a.g, u.l, u.s, u.h);
  const int budget = a.g.budget;
  const int esize = a.row_bytes / a.g.d;
  uint8_t* base = reinterpret_cast<uint8_t*>(which ? a.v : a.k) + (tid % TPR) * 16;
  const int rr = tid / TPR;
  const int32_t* krow = a.keep + out_row(a.g, u) * budget;

  if (tid == 0) first_moved = budget;
  __syncthreads();
  int lo = budget;
  for (int i = tid; i < budget; i += NT) {
    const int src = krow[i];
    keep_s[i] = src;
    if (src != i) lo = min(lo, i);
  }
  if (lo < budget) atomicMin(&first_moved, lo);
  __syncthreads();
  const int start = first_moved;

  // a tile's writes are still in flight while the next tile's reads go out;
  // the wait before each barrier covers both.  The tile lives in named
  // registers (an array here would be kept in scratch across the barrier).
  for (int t0 = start; t0 < budget; t0 += TILE) {
#define RKV_LOAD(r)                                                                  \
    const int s##r = min(t0 + r * RPP + rr, budget - 1);                             \
    const uint4 b##r = stream_load(reinterpret_cast<const uint4*>(                   \
        base + row_at<PAGED>(a, u, hb, keep_s[s##r]) * esize));
#define RKV_STORE(r) stream_store(reinterpret_cast<uint4*>(base + row_at<PAGED>(a, u, hb, s##r) * esize), b##r);
    static_assert(R == 8, "eight named row registers");
    RKV_LOAD(0) RKV_LOAD(1) RKV_LOAD(2) RKV_LOAD(3) RKV_LOAD(4) RKV_LOAD(5) RKV_LOAD(6) RKV_LOAD(7)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    RKV_STORE(0) RKV_STORE(1) RKV_STORE(2) RKV_STORE(3)
    RKV_STORE(4) RKV_STORE(5) RKV_STORE(6) RKV_STORE(7)
#undef RKV_LOAD
#undef RKV_STORE
  }

  if (a.free_blocks != nullptr && which == 0 && u.l == 0 && u.h == 0) {
    const int bs = 1 << a.g.bs_shift;
    const int first = (budget + bs - 1) / bs, last = (u.n + bs - 1) / bs;
    int32_t* out = a.free_blocks + free_off(a.g, a.tt, u.ti);
    for (int b = first + tid; b < last; b += NT)
      out[b - first] = a.bt[(int64_t)u.s * a.g.maxblk + b];
  }
}

template <bool PAGED, int TPR>
hipError_t launch_compact_t(const CompactArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (lds > 48 * 1024) {
    static const hipError_t once = hipFuncSetAttribute(
        reinterpret_cast<const void*>(compact_kernel<PAGED, TPR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, RKV_MAX_LEN * (int)sizeof(int32_t));
    if (once != hipSuccess) return once;
  }
  hipLaunchKernelGGL((compact_kernel<PAGED, TPR>), grid, dim3(kCompactThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid(units * 2);
  const size_t lds = (size_t)a.g.budget * sizeof(int32_t);
  // whole rows of 128, 256 or 512 bytes per workgroup
  switch (a.row_bytes) {
    case 128: return a.g.paged ? launch_compact_t<true, 8>(a, grid, lds, st) : launch_compact_t<false, 8>(a, grid, lds, st);
    case 256: return a.g.paged ? launch_compact_t<true, 16>(a, grid, lds, st) : launch_compact_t<false, 16>(a, grid, lds, st);
    case 512: return a.g.paged ? launch_compact_t<true, 32>(a, grid, lds, st) : launch_compact_t<false, 32>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rkv
