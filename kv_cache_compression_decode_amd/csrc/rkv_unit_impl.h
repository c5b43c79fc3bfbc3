// Single-pass scoring for units of up to 16 * 16 * NBW keys (1280 at
// head_dim 128): one 1024-thread workgroup per unit keeps all of the unit's
// keys in registers, so the keys are read from HBM once (the two-kernel
// path in rkv_score_impl.h reads them twice).  Same quantities as that path
// (R-KV project page on hysenlabs.com, "How R-KV decides what to drop";
// hotdry blog post, R-KV section):
//   I_j = (1/(G w)) sum_r exp(y_rj - m_r) / Z_r,  R_j = (khat_j . sum khat - 1)/(N - 1),
//   S_j = lambda I_j - (1 - lambda) R_j.
// Phases, each over the register-resident key fragments:
//   1. 1/|k| per key and the unit's sum of khat (DPP row sums, LDS across waves)
//   2. per window row, the max of y = q.k scaled and the sum of exp2(y - max)
//      (keys x rows MFMA; per chunk of key blocks the max first, then the sum)
//   3. rows x keys MFMA with the sum of khat as two extra bf16 rows: first
//      the redundancy (tiles holding the sum rows), then the importance
//      (window tiles) and the mixed score.
// Window-query rows live in LDS with a padded row pitch (D + 8 elements) so
// the 16 rows a fragment read touches fall in different banks.
#pragma once

#include "rkv_score_impl.h"

namespace rkv {

constexpr int kUnitWaves = 16;
constexpr int kUnitThreads = kUnitWaves * kWave;

template <int D>
struct UnitShape {
  static constexpr int NBW = D == 128 ? 5 : 10;              // 16-key blocks per wave
  static constexpr int NMAX = kUnitWaves * NBW * kBlockKeys;  // longest unit
};

// LDS of the single-pass scoring.
template <int D, int RT>
struct UnitLds {
  static constexpr int QP = D + 8;                 // row pitch of the window rows (elements)
  // 16-byte pieces of the window rows, one per thread per round; the extra
  // row only absorbs the stores of threads without a piece
  static constexpr int QITEMS = RT * 16 * (D / 8);
  static constexpr int QPER = (QITEMS + kUnitThreads - 1) / kUnitThreads;
  __attribute__((aligned(16))) uint16_t q[(RT * 16 + 1) * QP];
  // per-wave partials, wave index last: the 16 lanes that merge one row (or
  // one dim) read 16 consecutive words
  float red_m[RT * 16][kUnitWaves];
  float red_z[RT * 16][kUnitWaves];
  float red_s[D][kUnitWaves];
  float row_m[RT * 16], row_iz[RT * 16];
  float rn[UnitShape<D>::NMAX];                    // 1/|k| per key, then R_j
};

// Points at which unit_score calls its prefetch hook, once each, after the
// keys are on chip: 0 after phase 2, 1 before phase 3, 2 before its
// importance part, 3 after it.  A caller streaming memory that overlaps the
// arithmetic spreads its loads over them, so that no wave waits long for
// room to issue a load.
constexpr int kPrefetchStages = 4;

// Loads keys [k0, k0 + nl) of the unit into kf (blocks wave + 16 j of the
// span) and scores them; calls prefetch(stage) at the points above and
// sink(key, S_j) once per key of the span (index within the span) from the
// lane that holds it (after writing the score outputs).  All kUnitThreads
// threads call it.  SPAN = false: the span is the whole unit.  SPAN = true:
// the unit is split over several workgroups; after the span's own row
// statistics and direction sum are in LDS (row_m, row_iz = the span's raw
// sum, red_s[d][0]), exchange() must replace them by the unit's: row_m,
// row_iz as below and the two direction-sum rows of q.
template <bool PAGED, int D, int RT, bool SPAN, typename Prefetch, typename Sink,
          typename Exchange>
__device__ __forceinline__ void unit_score_span(const ScoreArgs& a, const Unit& u, int k0, int nl,
                                                UnitLds<D, RT>& L,
                                                KeyFrag<true, D> (&kf)[UnitShape<D>::NBW],
                                                Prefetch prefetch, Sink sink, Exchange exchange) {
  constexpr int KS = D / 32;
  constexpr int NBW = UnitShape<D>::NBW;
  constexpr int QP = UnitLds<D, RT>::QP;
  uint16_t* q_lds = L.q;
  auto& red_m = L.red_m;
  auto& red_z = L.red_z;
  auto& red_s = L.red_s;
  float* row_m = L.row_m;
  float* row_iz = L.row_iz;
  float* rn_lds = L.rn;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int t = threadIdx.x;
  const int n = nl;           // keys of the span
  const int gw = a.gw, rt1 = (gw + 15) >> 4;
  // Loads are unconditional (addresses clamped into the unit) so that no
  // branch makes a wave wait on one load before issuing the next.  The
  // window rows go first: writing them to LDS then waits for them only.
  constexpr int QPER = UnitLds<D, RT>::QPER;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + q_offset(a, u);
  uint4 qv[QPER];
#pragma unroll
  for (int p = 0; p < QPER; ++p) {
    const int i = t + p * kUnitThreads;
    const int r = min(i / (D / 8), gw - 1), c8 = i % (D / 8);
    qv[p] = *reinterpret_cast<const uint4*>(q + (int64_t)r * D + 8 * c8);
  }
  __builtin_amdgcn_sched_barrier(0);   // window-row loads issue before the key loads
  // keys of blocks wave + 16 j into registers; a lane past the end loads the
  // unit's last key, which every later use masks out.  The first KE blocks
  // are requested before the barrier that publishes the window rows, the
  // rest after it, so that barrier is not held up by waves still waiting for
  // room to issue loads, and each wave starts phases 1-2 as soon as its own
  // keys arrive.  (Paged rows need block-table loads for their addresses;
  // waiting for those after the barrier would also wait for the keys already
  // requested, so the paged layout requests every block first.)
  constexpr int KE = PAGED ? NBW : (NBW < 2 ? NBW : 2);
  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
    kf[j].load(a.k, rows.at(k0 + min(key, n - 1)), g4, true);
  }
  // window rows into LDS; rows >= gw are zero until the sum rows are written
#pragma unroll
  for (int p = 0; p < QPER; ++p) {
    const int i = t + p * kUnitThreads;
    const int r = min(i / (D / 8), RT * 16), c8 = i % (D / 8);
    const uint4 v = r < gw ? qv[p] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(q_lds + r * QP + 8 * c8) = v;
  }
  lds_barrier();   // window rows in LDS
#pragma unroll
  for (int j = KE; j < NBW; ++j) {
    const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
    kf[j].load(a.k, rows.at(k0 + min(key, n - 1)), g4, true);
  }

  // 1. 1/|k| and the sum of khat
  float rn[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const float n2 = sum_rows(kf[j].sq_norm_part());
    const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
    rn[j] = key < n && n2 > 0.f ? fast_rsqrt(n2) : 0.f;
    if (g4 == 0 && key < n) rn_lds[key] = rn[j];
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float s8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = 0.f;
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) s8[e] = fmaf(rn[j], kf[j].at(ks, e), s8[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = sum_in_row(s8[e]);
    if (col == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_s[32 * ks + 8 * g4 + e][wave] = s8[e];
    }
  }

  // the wave's key blocks that hold a key: blocks wave + 16 j, j < nbl
  const int nbl = __builtin_amdgcn_readfirstlane((n - wave * kBlockKeys + kUnitWaves * kBlockKeys - 1) /
                                                 (kUnitWaves * kBlockKeys));
  // 2. per window row, the max of y = q.k scaled (log2 units) and the sum of
  // exp2(y - max) over the wave's keys (keys x rows: lane holds keys
  // 4*g4 + i of row col).  Key blocks are taken PH2 at a time: all products
  // of a chunk are formed before any exponential, so the chunk's row max is
  // known first and the running sum is rescaled once per chunk.  The
  // exponent is one fma of the raw product: exp2(p * c - max).  Blocks past
  // the unit's end are skipped (a wave-uniform test).  Keys past the end in
  // a lane's last block were loaded as copies of the last key: they leave
  // the max unchanged, and the sum leaves them out.
  constexpr int PH2 = NBW < 2 ? NBW : 2;   // more live products spill registers
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (rt >= rt1) continue;
    float mx = -INFINITY, zz = 0.f;
    bf16x8 qf[KS];   // the tile's rows, read once for all key blocks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rt * 16 + col) * QP + 32 * ks + 8 * g4);
#pragma unroll
    for (int j0 = 0; j0 < NBW; j0 += PH2) {
      if (j0 >= nbl) continue;
      bool live[PH2];
#pragma unroll
      for (int j = 0; j < PH2; ++j) live[j] = j0 + j < NBW && j0 + j < nbl;
      f32x4 c[PH2];
#pragma unroll
      for (int j = 0; j < PH2; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {   // one 32-dim slice of the rows at a time
#pragma unroll
        for (int j = 0; j < PH2; ++j)
          if (live[j])
            c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, kf[j0 + j].w[ks]), qf[ks], c[j], 0, 0, 0);
      }
      float cm = -INFINITY;   // max of the raw products (the scale a.c > 0 keeps the order)
#pragma unroll
      for (int j = 0; j < PH2; ++j)
        if (live[j])
#pragma unroll
          for (int i = 0; i < 4; ++i) cm = fmaxf(cm, c[j][i]);
      const float mn = fmaxf(mx, xmax32(xmax16(cm)));   // same on the 4 lanes of the row
      const float off = mn * a.c;                        // log2 units; finite: a key is live
      float zc = 0.f;
#pragma unroll
      for (int j = 0; j < PH2; ++j) {
        if (!live[j]) continue;
        const int nv = n - (wave + kUnitWaves * (j0 + j)) * kBlockKeys - 4 * g4;   // valid of the 4
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(c[j][i], a.c, -off));
          zc += i < nv ? e : 0.f;
        }
      }
      zz = j0 == 0 ? zc : fmaf(zz, fast_exp2(fmaf(mx, a.c, -off)), zc);
      mx = mn;
    }
    zz = sum_rows(zz);
    if (g4 == 0) {
      red_m[rt * 16 + col][wave] = mx == -INFINITY ? mx : mx * a.c;   // log2 units
      red_z[rt * 16 + col][wave] = zz;
    }
  }
  lds_barrier();   // every wave's partials in LDS
  prefetch(0);
  // the waves' partials merged by rows of 16 lanes (lane = wave): per
  // window row the max and the rescaled sum; per dim the sum of khat, split
  // into the two bf16 rows gw and gw + 1.  Trip counts are wave-uniform
  // (RT * 256 and D * 16 are multiples of 64).
  static_assert(kUnitWaves == 16, "one DPP row of lanes per merged row");
  for (int idx = t; idx < RT * 16 * kUnitWaves; idx += kUnitThreads) {
    const int r = idx / kUnitWaves, w = idx % kUnitWaves;
    const float m = r < gw ? red_m[r][w] : -INFINITY;
    const float mm = max_in_row(m);
    const float z = sum_in_row(mm == -INFINITY ? 0.f : red_z[r][w] * fast_exp2(m - mm));
    if (w == 0) {
      if (SPAN) {
        row_m[r] = mm;
        row_iz[r] = z;
      } else {
        row_m[r] = r < gw ? mm : INFINITY;   // log2 units; other rows add nothing
        row_iz[r] = r < gw ? 1.f / (z * (float)gw) : 0.f;
      }
    }
  }
  for (int idx = t; idx < D * kUnitWaves; idx += kUnitThreads) {
    const int d = idx / kUnitWaves, w = idx % kUnitWaves;
    const float sv = sum_in_row(red_s[d][w]);   // the row group read all 16 before this write
    if (w == 0) {
      if (SPAN) {
        red_s[d][0] = sv;
      } else {
        const uint32_t hi = f2bf_bits(sv);
        q_lds[gw * QP + d] = (uint16_t)hi;
        q_lds[(gw + 1) * QP + d] = (uint16_t)f2bf_bits(sv - __uint_as_float(hi << 16));
      }
    }
  }
  if (SPAN) exchange();
  lds_barrier();

  prefetch(1);
  // 3. rows x keys (lane holds rows 4*g4 + i of key col).
  // 3a: the tile(s) holding the sum rows give khat . sum khat, hence the
  // redundancy, which replaces 1/|k| in LDS.
  const int st0 = gw >> 4, st1 = (gw + 1) >> 4;
  const float inv_nm1 = 1.f / (float)(u.n - 1);   // the whole unit's N
  {
    float sd[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) sd[j] = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt != st0 && rt != st1) continue;
      bf16x8 qf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rt * 16 + col) * QP + 32 * ks + 8 * g4);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        if (j >= nbl) continue;   // past the end (wave-uniform)
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], __builtin_bit_cast(bf16x8, kf[j].w[ks]),
                                                      c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * g4 + i;
          if (r == gw || r == gw + 1) sd[j] += c[i];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const float sdj = sum_rows(sd[j]);
      const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
      if (g4 == 0 && key < n) {
        const float rk = rn_lds[key];
        rn_lds[key] = rk > 0.f ? (sdj * rk - 1.f) * inv_nm1 : 0.f;   // now R_j
      }
    }
  }
  prefetch(2);
  // 3b: the window tiles give the importance; then the mixed score.
  float ip[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) ip[j] = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (rt >= rt1) continue;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rt * 16 + col) * QP + 32 * ks + 8 * g4);
    float mr[4], iz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mr[i] = row_m[rt * 16 + 4 * g4 + i];
      iz[i] = row_iz[rt * 16 + 4 * g4 + i];
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      if (j >= nbl) continue;   // past the end (wave-uniform)
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], __builtin_bit_cast(bf16x8, kf[j].w[ks]),
                                                    c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) ip[j] = fmaf(fast_exp2(fmaf(c[i], a.c, -mr[i])), iz[i], ip[j]);
    }
  }
  prefetch(3);
  const int64_t orow = out_row(a.g, u) * a.score_stride;
  float* const s_row = a.scores + orow;
  float* const i_row = a.imp != nullptr ? a.imp + orow : nullptr;
  float* const r_row = a.red != nullptr ? a.red + orow : nullptr;
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const float ipj = sum_rows(ip[j]);
    const int key = (wave + kUnitWaves * j) * kBlockKeys + col;
    if (g4 == 0 && key < n) {
      const float red = rn_lds[key];
      const float sc = a.lambda * ipj - (1.f - a.lambda) * red;
      s_row[k0 + key] = sc;
      if (i_row) i_row[k0 + key] = ipj;
      if (r_row) r_row[k0 + key] = red;
      sink(key, sc);
    }
  }
}

template <bool PAGED, int D, int RT, typename Prefetch, typename Sink>
__device__ __forceinline__ void unit_score(const ScoreArgs& a, const Unit& u, UnitLds<D, RT>& L,
                                           KeyFrag<true, D> (&kf)[UnitShape<D>::NBW],
                                           Prefetch prefetch, Sink sink) {
  unit_score_span<PAGED, D, RT, false>(a, u, 0, u.n, L, kf, prefetch, sink, [] {});
}

template <bool PAGED, int D, int RT>
__global__ __launch_bounds__(kUnitThreads) void score_unit_kernel(ScoreArgs a) {
  __shared__ UnitLds<D, RT> L;
  KeyFrag<true, D> kf[UnitShape<D>::NBW];
  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  if (u.n == 0) return;   // past the device table's count
  if (a.reset_status) clear_status_first(a.status);
  if (a.check_blocks && step_aborted(a.status, kBadBlockId)) return;   // the pool must not be read
  unit_score<PAGED, D, RT>(a, u, L, kf, [](int) {}, [](int, float) {});
}


template <bool PAGED, int D, int RT>
hipError_t launch_unit_t(const ScoreArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((score_unit_kernel<PAGED, D, RT>), dim3(units), dim3(kUnitThreads), 0, st, a);
  return hipGetLastError();
}

// Window + sum rows up to 5 tiles (G * w <= 78) take the single-pass kernel.
constexpr int kUnitMaxRowTiles = 5;

template <bool PAGED, int D>
hipError_t dispatch_unit(const ScoreArgs& a, int units, int rt2, hipStream_t st) {
  typedef hipError_t (*Fn)(const ScoreArgs&, int, hipStream_t);
  static const Fn fns[kUnitMaxRowTiles] = {launch_unit_t<PAGED, D, 1>, launch_unit_t<PAGED, D, 2>,
                                           launch_unit_t<PAGED, D, 3>, launch_unit_t<PAGED, D, 4>,
                                           launch_unit_t<PAGED, D, 5>};
  return fns[rt2 - 1](a, units, st);
}

}  // namespace rkv
