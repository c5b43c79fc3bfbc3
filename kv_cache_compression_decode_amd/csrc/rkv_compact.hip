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
// (phase 2).  Reads of the next tile touch rows >= its first slot, which no
// earlier tile writes, so the next tile's reads overlap this tile's writes.
// Slots with keep[i] == i are neither read nor written.
//
// One workgroup per (unit, K or V); 16 bytes per lane per row access, rows
// of 256 bytes read by 16 consecutive lanes.
#include "rkv_device.h"
#include "rkv_launch.h"

namespace rkv {

template <int TPR, int R>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  constexpr int RPP = kThreads / TPR;   // rows per pass
  constexpr int TILE = RPP * R;         // rows per phase-1/phase-2 round
  const int unit_id = blockIdx.x >> 1, which = blockIdx.x & 1;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  const int tid = threadIdx.x;
  const int sub = tid % TPR, rr = tid / TPR;
  const int budget = a.g.budget;
  const int esize = a.row_bytes / a.g.d;
  uint8_t* base = reinterpret_cast<uint8_t*>(which ? a.v : a.k);
  const int32_t* krow = a.keep + out_row(a.g, u) * budget;

  for (int i0 = 0; i0 < budget; i0 += TILE) {
    uint4 buf[R];
    int slot[R];
    bool mv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      slot[r] = i0 + r * RPP + rr;
      mv[r] = false;
      if (slot[r] < budget) {
        const int src = krow[slot[r]];
        mv[r] = src != slot[r];
        if (mv[r]) {
          const int64_t off = row_offset(a.g, a.bt, u.l, u.s, u.h, src) * esize + sub * 16;
          buf[r] = *reinterpret_cast<const uint4*>(base + off);
        }
      }
    }
    // every read of this tile has returned before any lane writes
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (mv[r]) {
        const int64_t off = row_offset(a.g, a.bt, u.l, u.s, u.h, slot[r]) * esize + sub * 16;
        *reinterpret_cast<uint4*>(base + off) = buf[r];
      }
    }
  }

  if (a.free_blocks != nullptr && which == 0 && u.l == 0 && u.h == 0) {
    const int bs = 1 << a.g.bs_shift;
    const int first = (budget + bs - 1) / bs, last = (u.n + bs - 1) / bs;
    int32_t* out = a.free_blocks + a.tt.free_off[u.ti];
    for (int b = first + tid; b < last; b += kThreads)
      out[b - first] = a.bt[(int64_t)u.s * a.g.maxblk + b];
  }
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid(units * 2);
  switch (a.row_bytes) {
    case 128: hipLaunchKernelGGL((compact_kernel<8, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 256: hipLaunchKernelGGL((compact_kernel<16, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 512: hipLaunchKernelGGL((compact_kernel<32, 4>), grid, dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rkv
