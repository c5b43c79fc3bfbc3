// Table of triggered sequences built on the GPU from device-resident
// lengths (rkv_step_device): the decode-time trigger of the R-KV project page
// ("How R-KV decides what to drop": compress once a sequence's cache reaches
// budget + buffer) taken without a host round trip, so that the whole step
// can run inside a captured decode graph.  One 1024-thread workgroup walks
// the sequences in order, 1024 at a time; two workgroup scans give each
// triggered sequence its table row and its first FREE_BLOCKS entry.
//
// Both kernels here also start the call's status word: they clear it, and
// with a block table to check they set kBadBlockId if a triggered sequence
// uses a block id outside [0, num_blocks) -- before any kernel of the call
// reads the pool.
#include "rkv_launch.h"
#include "rkv_select_impl.h"

namespace rkv {

constexpr int kTableThreads = 1024;

// All threads of one workgroup: is any of the n_blk first entries of row
// outside [0, nblk)?  (Each thread ORs its own findings into the status.)
__device__ __forceinline__ void check_block_row(const int32_t* row, int n_blk, int nblk,
                                                uint32_t* status) {
  bool bad = false;
  for (int b = threadIdx.x; b < n_blk; b += blockDim.x) bad |= (uint32_t)row[b] >= (uint32_t)nblk;
  if (bad) __hip_atomic_fetch_or(status, kBadBlockId, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void clear_status(uint32_t* status) {
  __hip_atomic_store(status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a) {
  if (a.reset && threadIdx.x == 0) clear_status(a.status);
  if (a.bt == nullptr) return;
  __syncthreads();   // the clear is done before any flag is set
  const int bs_shift = a.g.bs_shift;
  for (int ti = 0; ti < a.g.num_trig; ++ti) {
    const int n_blk = (a.tt.len[ti] + (1 << bs_shift) - 1) >> bs_shift;
    check_block_row(a.bt + (int64_t)a.tt.seq[ti] * a.g.maxblk, n_blk, a.g.nblk, a.status);
  }
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(prologue_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(kTableThreads) void table_kernel(TableArgs a) {
  __shared__ int tot_t[kTableThreads / kWave], tot_f[kTableThreads / kWave];
  __shared__ int base_t, base_f;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int S = a.num_seqs;
  const int kept_blocks = a.block_size > 0 ? (a.budget + a.block_size - 1) / a.block_size : 0;
  if (t == 0) {
    base_t = 0;
    base_f = 0;
    if (a.status != nullptr) clear_status(a.status);
  }
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += kTableThreads) {
    const int s = c0 + t;
    int n = 0, trig = 0, nf = 0;
    if (s < S) {
      n = a.lens[s];
      trig = n >= a.trigger && n <= a.max_len;   // longer than the launch bound: left alone
      if (trig && a.block_size > 0) nf = max(0, (n + a.block_size - 1) / a.block_size - kept_blocks);
    }
    const int it = wave_incl_scan(trig), inf = wave_incl_scan(nf);
    if (lane == kWave - 1) {
      tot_t[wave] = it;
      tot_f[wave] = inf;
    }
    __syncthreads();
    int bt = base_t, bf = base_f;
    for (int w = 0; w < wave; ++w) {
      bt += tot_t[w];
      bf += tot_f[w];
    }
    if (trig) {
      const int row = bt + it - 1;
      a.dtab[1 + row] = s;
      a.dtab[1 + S + row] = n;
      a.dtab[1 + 2 * S + row] = bf + inf - nf;
      a.lens[s] = a.budget;
    }
    if (s < S && a.free_counts != nullptr) a.free_counts[s] = nf;
    __syncthreads();   // every thread has read base_t / base_f
    if (t == kTableThreads - 1) {
      base_t = bt + it;
      base_f = bf + inf;
    }
    __syncthreads();
  }
  if (t == 0) a.dtab[0] = base_t;
  if (a.bt == nullptr) return;
  // the triggered sequences' block ids, from the table just written (the
  // barrier orders this workgroup's global writes before the reads)
  __syncthreads();
  const int count = base_t;
  for (int ti = 0; ti < count; ++ti) {
    const int s = a.dtab[1 + ti], n = a.dtab[1 + S + ti];
    check_block_row(a.bt + (int64_t)s * a.maxblk, (n + a.block_size - 1) / a.block_size, a.nblk,
                    a.status);
  }
}

hipError_t launch_table(const TableArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(table_kernel, dim3(1), dim3(kTableThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rkv
