// Scoring pass of the R-KV compression step: importance, redundancy and the
// mixed score of every cached token of every triggered unit, all layers in
// one launch pair ("batched cross-layer scoring", R-KV project page on
// hysenlabs.com, section "How R-KV decides what to drop"; the two signals
// and their blend: hotdry blog post, R-KV section).
//
// Per unit (sequence s, layer l, kv head h) with N keys k_j and the G*w
// window-query rows q_r of the G query heads sharing h:
//   I_j = (1/(G w)) sum_r exp(y_rj - m_r) / Z_r,   y_rj = q_r.k_j / sqrt(d)
//   R_j = (khat_j . sum_k khat_k - 1) / (N - 1),    khat = k / |k|
//   S_j = lambda I_j - (1 - lambda) R_j
// The redundancy is the mean off-diagonal entry of row j of the cosine Gram
// matrix; summing that row is the product of the Gram matrix with the ones
// vector, evaluated here in the order khat_j . (Khat^T 1), so the N x N
// matrix is never formed and the pass stays bandwidth-bound.
//
// Two kernels, one workgroup per (unit, 256-key chunk):
//   stats:    for its chunk, per window row the max and the sum of
//             exp2(y - max); per key 1/|k|; the chunk's sum of khat.  Written
//             to the workspace as one record per (unit, chunk).
//   finalize: merges the unit's records, then re-reads its chunk (from L2 /
//             infinity cache) and computes I, R, S.  The window-query
//             contraction and the khat . sum contraction share one bf16 MFMA
//             pass: the fp32 direction sum is split into two bf16 rows
//             (hi + lo) appended below the query rows.
// Keys go straight from global memory into MFMA operand registers: lane l
// loads, for key (l & 15) of a 16-key block, dims 32 ks + 8 (l >> 4) .. +7,
// which is both the v_mfma_f32_16x16x32_bf16 B-operand layout and 64
// contiguous bytes per key per instruction.
#pragma once

#include <math.h>

#include "rkv_device.h"
#include "rkv_launch.h"

namespace rkv {

namespace detail {

template <int KS>
struct KFrag {
  uint4 w[KS];   // bf16: 8 values per uint4; f32 path uses two KFrags
};

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// Merge two (max, sum-of-exp2) pairs expressed in log2 units.
__device__ __forceinline__ void merge_stats(float& m, float& z, float m2, float z2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    z = 0.f;
    return;
  }
  z = z * exp2f(m - mm) + z2 * exp2f(m2 - mm);
  m = mm;
}

// ---------------------------------------------------------------- key loads
// bf16: uint4 x KS per lane.  f32: the same dims as two float4 per k-step.
template <bool BF16, int D>
struct KeyFrag;

template <int D>
struct KeyFrag<true, D> {
  static constexpr int KS = D / 32;
  uint4 w[KS];
  __device__ __forceinline__ void load(const void* base, int64_t row, int g4, bool valid) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + row + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      w[ks] = valid ? *reinterpret_cast<const uint4*>(p + 32 * ks) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ float sq_norm_part() const {
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t v[4] = {w[ks].x, w[ks].y, w[ks].z, w[ks].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v[j]),
                                              __builtin_bit_cast(bf16x2, v[j]), acc, false);
    }
    return acc;
  }
  // element e (0..7) of k-step ks as float
  __device__ __forceinline__ float at(int ks, int e) const {
    const uint32_t v[4] = {w[ks].x, w[ks].y, w[ks].z, w[ks].w};
    return (e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1]);
  }
};

template <int D>
struct KeyFrag<false, D> {
  static constexpr int KS = D / 32;
  float4 w[KS][2];
  __device__ __forceinline__ void load(const void* base, int64_t row, int g4, bool valid) {
    const float* p = reinterpret_cast<const float*>(base) + row + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      w[ks][0] = valid ? *reinterpret_cast<const float4*>(p + 32 * ks) : make_float4(0, 0, 0, 0);
      w[ks][1] = valid ? *reinterpret_cast<const float4*>(p + 32 * ks + 4) : make_float4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ float at(int ks, int e) const {
    const float4 v = w[ks][e >> 2];
    const int i = e & 3;
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ float sq_norm_part() const {
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(at(ks, e), at(ks, e), acc);
    return acc;
  }
};

// ---------------------------------------------------------------- query operand
// bf16: A-operand registers of RT row tiles.  f32: rows staged in LDS.
template <bool BF16, int D, int RT>
struct QOperand;

template <int D, int RT>
struct QOperand<true, D, RT> {
  static constexpr int KS = D / 32;
  bf16x8 a[RT][KS];
  // rows < gw from q (bf16), row gw / gw+1 = hi / lo bf16 parts of s (if s != nullptr)
  __device__ __forceinline__ void load(const uint16_t* q, int gw, const float* s_lds, int lane) {
    const int col = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < gw) {
          v = *reinterpret_cast<const uint4*>(q + (int64_t)r * D + 32 * ks + 8 * g4);
        } else if (s_lds != nullptr && (r == gw || r == gw + 1)) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sv = s_lds[32 * ks + 8 * g4 + e];
            const uint32_t hi = f2bf_bits(sv);
            h[e] = (r == gw) ? hi : f2bf_bits(sv - __uint_as_float(hi << 16));
          }
          v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16));
        }
        a[rt][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  // raw dot products: acc[rt][i] = row (rt*16 + 4*g4 + i) . key (lane & 15)
  __device__ __forceinline__ void logits(const KeyFrag<true, D>& k, float (&acc)[RT][4]) const {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][ks], __builtin_bit_cast(bf16x8, k.w[ks]),
                                                    c, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = c[i];
    }
  }
};

template <int D, int RT>
struct QOperand<false, D, RT> {
  static constexpr int KS = D / 32;
  const float* rows;   // LDS, RT*16 x D
  int lane;
  // the caller stages rows (q rows < gw, s at row gw, zeros elsewhere) in LDS
  __device__ __forceinline__ void bind(const float* lds_rows, int ln) {
    rows = lds_rows;
    lane = ln;
  }
  __device__ __forceinline__ void logits(const KeyFrag<false, D>& k, float (&acc)[RT][4]) const {
    const int g4 = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = 0.f;
#pragma unroll 1
      for (int rr = 0; rr < 16; ++rr) {
        const float* qr = rows + (rt * 16 + rr) * D + 8 * g4;
        float p = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(qr[32 * ks + e], k.at(ks, e), p);
        p += shfl_xor(p, 16);
        p += shfl_xor(p, 32);
        if ((rr >> 2) == g4) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((rr & 3) == i) acc[rt][i] = p;
        }
      }
    }
  }
};

__device__ __forceinline__ int64_t q_offset(const ScoreArgs& a, const Unit& u) {
  return (((int64_t)u.l * a.g.num_seqs + u.s) * a.g.hq + (int64_t)u.h * a.g.group) *
         a.g.window * a.g.d;
}

template <bool BF16, int D, int RT>
__device__ __forceinline__ void stage_rows_f32(const ScoreArgs& a, const Unit& u, float* lds,
                                               const float* s_lds) {
  const float* q = reinterpret_cast<const float*>(a.q) + q_offset(a, u);
  for (int i = threadIdx.x; i < RT * 16 * D; i += kThreads) {
    const int r = i / D, c = i % D;
    float v = 0.f;
    if (r < a.gw) v = q[(int64_t)r * D + c];
    else if (s_lds != nullptr && r == a.gw) v = s_lds[c];
    lds[i] = v;
  }
}

}  // namespace detail

using namespace detail;

// ---------------------------------------------------------------- kernel 1
template <bool BF16, int D, int RT>
__global__ __launch_bounds__(kThreads) void score_stats_kernel(ScoreArgs a) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int unit_id = blockIdx.x / a.max_chunks, chunk = blockIdx.x % a.max_chunks;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  const int key_base = chunk * kChunk;
  if (key_base >= u.n) return;

  __shared__ float red_m[4][RT * 16], red_z[4][RT * 16], red_s[4][D];
  __shared__ float q_lds[BF16 ? 1 : RT * 16 * D];

  QOperand<BF16, D, RT> qop;
  if constexpr (BF16) {
    qop.load(reinterpret_cast<const uint16_t*>(a.q) + q_offset(a, u), a.gw, nullptr, lane);
  } else {
    stage_rows_f32<BF16, D, RT>(a, u, q_lds, nullptr);
    __syncthreads();
    qop.bind(q_lds, lane);
  }

  KeyFrag<BF16, D> kf[kBlocksPerWave];
  bool valid[kBlocksPerWave];
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    const int key = key_base + (wave + 4 * b) * kBlockKeys + col;
    valid[b] = key < u.n;
    const int64_t row = valid[b] ? row_offset(a.g, a.bt, u.l, u.s, u.h, key) : 0;
    kf[b].load(a.k, row, g4, valid[b]);
  }

  float y[kBlocksPerWave][RT][4];
  float sacc[KS * 8];
#pragma unroll
  for (int i = 0; i < KS * 8; ++i) sacc[i] = 0.f;

#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    float acc[RT][4];
    qop.logits(kf[b], acc);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) y[b][rt][i] = valid[b] ? acc[rt][i] * a.c : -INFINITY;
    float n2 = kf[b].sq_norm_part();
    n2 += shfl_xor(n2, 16);
    n2 += shfl_xor(n2, 32);
    const float rn = (valid[b] && n2 > 0.f) ? rsqrtf(n2) : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc[ks * 8 + e] = fmaf(rn, kf[b].at(ks, e), sacc[ks * 8 + e]);
  }

  // per-lane stats over its blocks, then across the 16 lanes that share rows
  float m[RT][4], z[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = y[0][rt][i];
#pragma unroll
      for (int b = 1; b < kBlocksPerWave; ++b) mx = fmaxf(mx, y[b][rt][i]);
      float zz = 0.f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int b = 0; b < kBlocksPerWave; ++b) zz += exp2f(y[b][rt][i] - mx);
      }
      m[rt][i] = mx;
      z[rt][i] = zz;
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) {
        const float m2 = shfl_xor(m[rt][i], x), z2 = shfl_xor(z[rt][i], x);
        merge_stats(m[rt][i], z[rt][i], m2, z2);
      }
    }
#pragma unroll
  for (int i = 0; i < KS * 8; ++i)
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) sacc[i] += shfl_xor(sacc[i], x);

  if (col == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red_m[wave][rt * 16 + 4 * g4 + i] = m[rt][i];
        red_z[wave][rt * 16 + 4 * g4 + i] = z[rt][i];
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_s[wave][32 * ks + 8 * g4 + e] = sacc[ks * 8 + e];
  }
  __syncthreads();

  float* rec = a.part + ((int64_t)unit_id * a.max_chunks + chunk) * a.rec;
  const int t = threadIdx.x;
  if (t < a.gw) {
    float mm = red_m[0][t], zz = red_z[0][t];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_stats(mm, zz, red_m[w][t], red_z[w][t]);
    rec[t] = mm;
    rec[a.gw + t] = zz;
  }
  if (t < D) rec[2 * a.gw + t] = red_s[0][t] + red_s[1][t] + red_s[2][t] + red_s[3][t];
}

// ---------------------------------------------------------------- kernel 2
template <bool BF16, int D, int RT>
__global__ __launch_bounds__(kThreads) void score_finalize_kernel(ScoreArgs a) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int unit_id = blockIdx.x / a.max_chunks, chunk = blockIdx.x % a.max_chunks;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  const int key_base = chunk * kChunk;
  if (key_base >= u.n) return;

  __shared__ float row_m[RT * 16], row_iz[RT * 16], s_lds[D];
  __shared__ float q_lds[BF16 ? 1 : RT * 16 * D];

  // merge the unit's chunk records (fixed order: deterministic)
  const int nch = (u.n + kChunk - 1) / kChunk;
  const float* recs = a.part + (int64_t)unit_id * a.max_chunks * a.rec;
  const int t = threadIdx.x;
  if (t < RT * 16) {
    if (t < a.gw) {
      float mm = recs[t], zz = recs[a.gw + t];
      for (int c = 1; c < nch; ++c) merge_stats(mm, zz, recs[c * a.rec + t], recs[c * a.rec + a.gw + t]);
      row_m[t] = mm;
      row_iz[t] = 1.f / (zz * (float)a.gw);
    } else {
      row_m[t] = INFINITY;   // padding and direction-sum rows add nothing to I
      row_iz[t] = 0.f;
    }
  }
  if (t < D) {
    float sv = 0.f;
    for (int c = 0; c < nch; ++c) sv += recs[c * a.rec + 2 * a.gw + t];
    s_lds[t] = sv;
  }
  __syncthreads();

  QOperand<BF16, D, RT> qop;
  if constexpr (BF16) {
    qop.load(reinterpret_cast<const uint16_t*>(a.q) + q_offset(a, u), a.gw, s_lds, lane);
  } else {
    stage_rows_f32<BF16, D, RT>(a, u, q_lds, s_lds);
    __syncthreads();
    qop.bind(q_lds, lane);
  }

  float mr[RT][4], izr[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mr[rt][i] = row_m[rt * 16 + 4 * g4 + i];
      izr[rt][i] = row_iz[rt * 16 + 4 * g4 + i];
    }
  const int srow0 = a.gw, srow1 = BF16 ? a.gw + 1 : a.gw;

  KeyFrag<BF16, D> kf[kBlocksPerWave];
  bool valid[kBlocksPerWave];
  int keys[kBlocksPerWave];
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    keys[b] = key_base + (wave + 4 * b) * kBlockKeys + col;
    valid[b] = keys[b] < u.n;
    const int64_t row = valid[b] ? row_offset(a.g, a.bt, u.l, u.s, u.h, keys[b]) : 0;
    kf[b].load(a.k, row, g4, valid[b]);
  }

  const int64_t orow = out_row(a.g, u) * a.score_stride;
  const float inv_nm1 = 1.f / (float)(u.n - 1);
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    float acc[RT][4];
    qop.logits(kf[b], acc);
    float ip = 0.f, sd = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt * 16 < a.gw) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ip = fmaf(exp2f(fmaf(acc[rt][i], a.c, -mr[rt][i])), izr[rt][i], ip);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * g4 + i;
        if (r == srow0 || r == srow1) sd += acc[rt][i];
      }
    }
    float n2 = kf[b].sq_norm_part();
    ip += shfl_xor(ip, 16);
    ip += shfl_xor(ip, 32);
    sd += shfl_xor(sd, 16);
    sd += shfl_xor(sd, 32);
    n2 += shfl_xor(n2, 16);
    n2 += shfl_xor(n2, 32);
    if (g4 == 0 && valid[b]) {
      const float red = n2 > 0.f ? (sd * rsqrtf(n2) - 1.f) * inv_nm1 : 0.f;
      const float sc = a.lambda * ip - (1.f - a.lambda) * red;
      a.scores[orow + keys[b]] = sc;
      if (a.imp) a.imp[orow + keys[b]] = ip;
      if (a.red) a.red[orow + keys[b]] = red;
    }
  }
}

// ---------------------------------------------------------------- launch
template <bool BF16, int D, int RT>
hipError_t launch_stats_t(const ScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_stats_kernel<BF16, D, RT>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
template <bool BF16, int D, int RT>
hipError_t launch_final_t(const ScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_finalize_kernel<BF16, D, RT>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// Both kernels of the scoring pass for one (dtype, head_dim); rt1 / rt2 are
// the row tiles of the window rows and of the window rows + 2 sum rows.
template <bool BF16, int D>
hipError_t dispatch_score(const ScoreArgs& a, int grid, int rt1, int rt2, hipStream_t st) {
  typedef hipError_t (*Fn)(const ScoreArgs&, int, hipStream_t);
  static const Fn stats[9] = {launch_stats_t<BF16, D, 1>, launch_stats_t<BF16, D, 2>,
                              launch_stats_t<BF16, D, 3>, launch_stats_t<BF16, D, 4>,
                              launch_stats_t<BF16, D, 5>, launch_stats_t<BF16, D, 6>,
                              launch_stats_t<BF16, D, 7>, launch_stats_t<BF16, D, 8>,
                              launch_stats_t<BF16, D, 9>};
  static const Fn fin[9] = {launch_final_t<BF16, D, 1>, launch_final_t<BF16, D, 2>,
                            launch_final_t<BF16, D, 3>, launch_final_t<BF16, D, 4>,
                            launch_final_t<BF16, D, 5>, launch_final_t<BF16, D, 6>,
                            launch_final_t<BF16, D, 7>, launch_final_t<BF16, D, 8>,
                            launch_final_t<BF16, D, 9>};
  hipError_t e = stats[rt1 - 1](a, grid, st);
  if (e != hipSuccess) return e;
  return fin[rt2 - 1](a, grid, st);
}

hipError_t dispatch_score_bf16_d64(const ScoreArgs&, int, int, int, hipStream_t);
hipError_t dispatch_score_bf16_d128(const ScoreArgs&, int, int, int, hipStream_t);
hipError_t dispatch_score_f32_d64(const ScoreArgs&, int, int, int, hipStream_t);
hipError_t dispatch_score_f32_d128(const ScoreArgs&, int, int, int, hipStream_t);

}  // namespace rkv
