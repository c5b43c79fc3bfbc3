// Window-query ring of the decode loop (R-KV project page on hysenlabs.com,
// "How R-KV decides what to drop": the last window_size queries of a sequence
// score its cache).  Decode step t of sequence s writes the queries of every
// query head, for layers layer0 .. layer0 + count - 1, into slot t mod window
// of the ring [layers][seqs][q_heads][window][head_dim] that the scoring calls
// read.  After any window consecutive steps the ring holds exactly the last
// window queries; importance averages over the window rows, so the rotated
// order they sit in does not change it.
//
// One 16-byte piece per thread; the slot comes from the step counter in
// device memory, so the call takes no host decision on it and can sit inside
// a captured decode graph.
#include "rkv_launch.h"

namespace rkv {

namespace {

__global__ __launch_bounds__(kThreads) void window_store_kernel(WindowArgs a) {
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= a.pieces) return;
  const int ppr = a.row_bytes / 16;                  // pieces per query row
  const int64_t row = p / ppr;                       // (i, s, h), layer-major
  const int piece = (int)(p % ppr);
  const int h = (int)(row % a.hq);
  const int64_t is = row / a.hq;
  const int s = (int)(is % a.num_seqs), i = (int)(is / a.num_seqs);
  int slot = a.steps[s] % a.window;
  if (slot < 0) slot += a.window;
  const uint4 v = *reinterpret_cast<const uint4*>(a.q_step + row * a.row_bytes + 16 * piece);
  const int64_t drow = (((int64_t)(a.layer0 + i) * a.num_seqs + s) * a.hq + h) * a.window + slot;
  *reinterpret_cast<uint4*>(a.q_window + drow * a.row_bytes + 16 * piece) = v;
}

}  // namespace

hipError_t launch_window_store(const WindowArgs& a, hipStream_t st) {
  if (a.pieces == 0) return hipSuccess;
  const int64_t grid = (a.pieces + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(window_store_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace rkv
