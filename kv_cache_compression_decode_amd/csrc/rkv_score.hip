// Host launcher of the scoring pass: the single-pass kernel of
// rkv_unit_impl.h for bf16 units that fit on chip, the key-span kernel of
// rkv_long_impl.h for longer bf16 units, else the two kernels of
// rkv_score_impl.h (one translation unit per cache dtype, head_dim, layout).
#include <atomic>

#include "rkv_step_impl.h"

namespace rkv {

hipError_t dispatch_unit_bf16_d64_contig(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_unit_bf16_d64_paged(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_unit_bf16_d128_contig(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_unit_bf16_d128_paged(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_step_bf16_d64_contig(const StepArgs&, int, int, hipStream_t);
hipError_t dispatch_step_bf16_d64_paged(const StepArgs&, int, int, hipStream_t);
hipError_t dispatch_step_bf16_d128_contig(const StepArgs&, int, int, hipStream_t);
hipError_t dispatch_step_bf16_d128_paged(const StepArgs&, int, int, hipStream_t);
hipError_t dispatch_long_bf16_d64_contig(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_long_bf16_d64_paged(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_long_bf16_d128_contig(const ScoreArgs&, int, int, hipStream_t);
hipError_t dispatch_long_bf16_d128_paged(const ScoreArgs&, int, int, hipStream_t);

namespace {
std::atomic<int64_t> g_span_wait_ticks{100000000};   // 1 s at 100 MHz

int long_chunks(const ScoreArgs& a) {
  const int nmax = a.g.d == 64 ? UnitShape<64>::NMAX : UnitShape<128>::NMAX;
  return (a.max_len + nmax - 1) / nmax;
}
}  // namespace

void set_span_wait_ticks(int64_t ticks) { g_span_wait_ticks.store(ticks, std::memory_order_relaxed); }
int64_t span_wait_ticks() { return g_span_wait_ticks.load(std::memory_order_relaxed); }

bool score_single_pass(const ScoreArgs& a, bool bf16, int max_len) {
  const int rt2 = (a.gw + 2 + 15) / 16;
  const int nmax = a.g.d == 64 ? UnitShape<64>::NMAX : UnitShape<128>::NMAX;
  return bf16 && rt2 <= kUnitMaxRowTiles && max_len <= nmax;
}

hipError_t launch_score(const ScoreArgs& a, bool bf16, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  const int grid = units * a.max_chunks;
  if (grid == 0) return hipSuccess;
  const int rt1 = (a.gw + 15) / 16;
  const int rt2 = (a.gw + 2 + 15) / 16;
  if (score_single_pass(a, bf16, a.max_len)) {
    if (a.g.d == 64)
      return a.g.paged ? dispatch_unit_bf16_d64_paged(a, units, rt2, st)
                       : dispatch_unit_bf16_d64_contig(a, units, rt2, st);
    return a.g.paged ? dispatch_unit_bf16_d128_paged(a, units, rt2, st)
                     : dispatch_unit_bf16_d128_contig(a, units, rt2, st);
  }
  if (bf16 && rt2 <= kUnitMaxRowTiles) {
    // longer bf16 units: key spans of at most NMAX keys on C workgroups each
    const int chunks = long_chunks(a);
    if (a.g.d == 64)
      return a.g.paged ? dispatch_long_bf16_d64_paged(a, chunks, rt2, st)
                       : dispatch_long_bf16_d64_contig(a, chunks, rt2, st);
    return a.g.paged ? dispatch_long_bf16_d128_paged(a, chunks, rt2, st)
                     : dispatch_long_bf16_d128_contig(a, chunks, rt2, st);
  }
#define RKV_PICK(DT, D)                                                              \
  return a.g.paged ? dispatch_score_##DT##_d##D##_paged(a, grid, rt1, rt2, st)       \
                   : dispatch_score_##DT##_d##D##_contig(a, grid, rt1, rt2, st)
  if (bf16) {
    if (a.g.d == 64) RKV_PICK(bf16, 64);
    RKV_PICK(bf16, 128);
  }
  if (a.g.d == 64) RKV_PICK(f32, 64);
  RKV_PICK(f32, 128);
#undef RKV_PICK
}

// The fused kernel selects per unit, so head-shared selection runs the three kernels.
bool step_fusable(const ScoreArgs& a, bool bf16) {
  return !a.g.shared && score_single_pass(a, bf16, a.max_len);
}

hipError_t launch_step(const StepArgs& a, hipStream_t st) {
  const int units = a.s.g.num_trig * a.s.g.num_layers * a.s.g.hkv;
  if (units == 0) return hipSuccess;
  const int rt2 = (a.s.gw + 2 + 15) / 16;
  if (a.s.g.d == 64)
    return a.s.g.paged ? dispatch_step_bf16_d64_paged(a, units, rt2, st)
                       : dispatch_step_bf16_d64_contig(a, units, rt2, st);
  return a.s.g.paged ? dispatch_step_bf16_d128_paged(a, units, rt2, st)
                     : dispatch_step_bf16_d128_contig(a, units, rt2, st);
}

}  // namespace rkv
