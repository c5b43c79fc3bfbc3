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
//             exp2(y - max); the chunk's sum of khat.  One record per
//             (unit, chunk) in the workspace.
//   finalize: merges the unit's records, re-reads its chunk and computes I,
//             R, S.  Its workgroups take the chunks in reverse order within
//             each XCD, so the chunks the stats kernel read last are re-read
//             first, from that XCD's L2.
// Keys go from global memory straight into MFMA operand registers: lane l
// loads, for key (l & 15) of a 16-key block, dims 32 ks + 8 (l >> 4) .. +7 --
// the operand layout of v_mfma_f32_16x16x32_bf16 (and, element by element,
// of v_mfma_f32_16x16x4_f32 for fp32 caches) and 64 contiguous bytes per key
// per load.  The stats kernel multiplies keys x rows, so a lane holds four
// keys of one window row and the row statistics reduce mostly in registers;
// the finalize kernel multiplies rows x keys, so a lane holds one key's
// rows and the per-key sums need two cross-row swaps.  In the finalize
// product the fp32 direction sum rides along as two extra bf16 rows (hi and
// lo parts; one fp32 row for fp32 caches).
#pragma once

#include <math.h>

#include "rkv_device.h"
#include "rkv_launch.h"

namespace rkv {

namespace detail {

// ---------------------------------------------------------------- lane exchange
// Sum / max with the partner lane l ^ 16 and l ^ 32 (v_permlane{16,32}_swap:
// the two outputs hold the value of a lane and of its partner).
__device__ __forceinline__ float xsum16(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xmax16(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xmax32(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
// Sum over the 4 lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float sum_rows(float v) { return xsum32(xsum16(v)); }

// Sum over the 16 lanes of a row (DPP; every lane of the row gets the total).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_in_row(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);   // row_half_mirror
  v = dpp_add<0x140>(v);   // row_mirror
  return v;
}
// Max over the 16 lanes of a row, likewise.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true)));
}
__device__ __forceinline__ float max_in_row(float v) {
  return dpp_max<0x140>(dpp_max<0x141>(dpp_max<0x4E>(dpp_max<0xB1>(v))));
}

// 2^x and 1/sqrt(x) as single hardware instructions (v_exp_f32, v_rsq_f32).
// Arguments of the exponentials are <= 0 (logit minus its running max), so
// results below 2^-126, flushed to zero, are negligible next to the max term.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// Merge two (max, sum of exp2(x - max)) pairs in log2 units.
__device__ __forceinline__ void merge_stats(float& m, float& z, float m2, float z2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    z = 0.f;
    return;
  }
  z = z * fast_exp2(m - mm) + z2 * fast_exp2(m2 - mm);
  m = mm;
}

// Merge (m0, z0) and (m1, z1) into (m, z); symmetric in its two pairs, so
// partner lanes that merge each other's stats get identical results.
__device__ __forceinline__ void merge_stats_pair(float m0, float z0, float m1, float z1, float& m,
                                                 float& z) {
  const float mm = fmaxf(m0, m1);
  m = mm;
  z = mm == -INFINITY ? 0.f : z0 * fast_exp2(m0 - mm) + z1 * fast_exp2(m1 - mm);
}

// ---------------------------------------------------------------- key operand
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
  __device__ __forceinline__ uint32_t word(int ks, int j) const {
    return j == 0 ? w[ks].x : j == 1 ? w[ks].y : j == 2 ? w[ks].z : w[ks].w;
  }
  __device__ __forceinline__ float at(int ks, int e) const {
    const uint32_t v = word(ks, e >> 1);
    return (e & 1) ? bf_hi(v) : bf_lo(v);
  }
  __device__ __forceinline__ float sq_norm_part() const {
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word(ks, j)),
                                              __builtin_bit_cast(bf16x2, word(ks, j)), acc, false);
    return acc;
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

// ---------------------------------------------------------------- row operand
// Window-query rows (+ direction-sum rows in the finalize kernel), RT tiles
// of 16 rows.  bf16: MFMA operand registers.  fp32: rows staged in LDS.
template <bool BF16, int D, int RT>
struct RowOp;

template <int D, int RT>
struct RowOp<true, D, RT> {
  static constexpr int KS = D / 32;
  bf16x8 a[RT][KS];
  // rows < gw from q; with s_hi / s_lo (LDS, bf16), rows gw and gw+1 hold them
  __device__ __forceinline__ void load(const uint16_t* q, int gw, const uint16_t* s_hi,
                                       const uint16_t* s_lo, int lane) {
    const int col = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = rt * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < gw)
          v = *reinterpret_cast<const uint4*>(q + (int64_t)r * D + 32 * ks + 8 * g4);
        else if (s_hi != nullptr && r <= gw + 1)
          v = *reinterpret_cast<const uint4*>((r == gw ? s_hi : s_lo) + 32 * ks + 8 * g4);
        a[rt][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  // TRANS: lane holds C[key 4*g4+i][row col]; else C[row 4*g4+i][key col]
  template <bool TRANS>
  __device__ __forceinline__ f32x4 tile(const KeyFrag<true, D>& k, int rt) const {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, k.w[ks]);
      c = TRANS ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, a[rt][ks], c, 0, 0, 0)
                : __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][ks], kb, c, 0, 0, 0);
    }
    return c;
  }
};

template <int D, int RT>
struct RowOp<false, D, RT> {
  static constexpr int KS = D / 32;
  const float* rows;   // LDS, RT*16 rows of D floats
  int col, g4;
  __device__ __forceinline__ void bind(const float* lds_rows, int lane) {
    rows = lds_rows;
    col = lane & 15;
    g4 = lane >> 4;
  }
  template <bool TRANS>
  __device__ __forceinline__ f32x4 tile(const KeyFrag<false, D>& k, int rt) const {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    const float* r = rows + (rt * 16 + col) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qv = r[32 * ks + e], kv = k.at(ks, e);
        c = TRANS ? __builtin_amdgcn_mfma_f32_16x16x4f32(kv, qv, c, 0, 0, 0)
                  : __builtin_amdgcn_mfma_f32_16x16x4f32(qv, kv, c, 0, 0, 0);
      }
    return c;
  }
};

__device__ __forceinline__ int64_t q_offset(const ScoreArgs& a, const Unit& u) {
  return (((int64_t)u.l * a.g.num_seqs + u.s) * a.g.hq + (int64_t)u.h * a.g.group) *
         a.g.window * a.g.d;
}

// Element offset of key t of one unit, relative to the unit's base.
template <bool PAGED>
struct KeyRows {
  int64_t base;          // element offset of the unit's row 0 (contiguous) / of its head in block 0
  const int32_t* bt;     // paged: the sequence's block-table row
  int64_t blk_stride;    // paged: elements per block of one layer
  int shift, d;
  __device__ __forceinline__ void init(const Geom& g, const int32_t* table, const Unit& u) {
    d = g.d;
    base = head_base(g, u.l, u.s, u.h);
    if constexpr (PAGED) {
      shift = g.bs_shift;
      blk_stride = ((int64_t)g.hkv << g.bs_shift) * g.d;
      bt = table + (int64_t)u.s * g.maxblk;
    }
  }
  __device__ __forceinline__ int64_t at(int t) const {
    if constexpr (PAGED)
      return base + bt[t >> shift] * blk_stride + (int64_t)(t & ((1 << shift) - 1)) * d;
    else
      return base + (int64_t)t * d;
  }
};

// fp32 caches: window rows, then (finalize) the direction sum as row gw.
template <int D, int RT>
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

// Work item of a finalize workgroup: the stats kernel's items in reverse
// order within each XCD (workgroup b runs on XCD b % 8).
__device__ __forceinline__ int finalize_item(int b, int grid) {
  const int x = b & 7, q = b >> 3;
  const int per = (grid - x + 7) >> 3;      // workgroups of this XCD
  return ((per - 1 - q) << 3) + x;
}

// Key fragments of the wave's blocks; missing keys (past N) load as zeros.
template <bool BF16, bool PAGED, int D, bool FULL>
__device__ __forceinline__ void load_keys(const ScoreArgs& a, const Unit& u, int chunk,
                                          KeyFrag<BF16, D> (&kf)[kBlocksPerWave]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
#pragma unroll
  for (int b = 0; b < kBlocksPerWave; ++b) {
    const int key = chunk * kChunk + (wave + 4 * b) * kBlockKeys + col;
    const bool valid = FULL || key < u.n;
    kf[b].load(a.k, valid ? rows.at(key) : 0, g4, valid);
  }
}

// ---------------------------------------------------------------- stats body
// FULL: every key of the chunk exists (no masking).
template <bool BF16, bool PAGED, int D, int RT, bool FULL>
__device__ __forceinline__ void stats_body(const ScoreArgs& a, const Unit& u, int unit_id, int chunk,
                                           float (*red_m)[RT * 16], float (*red_z)[RT * 16],
                                           float (*red_s)[D], float* q_lds) {
  constexpr int KS = D / 32;
  constexpr int NB = kBlocksPerWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int key_base = chunk * kChunk;

  KeyFrag<BF16, D> kf[NB];
  load_keys<BF16, PAGED, D, FULL>(a, u, chunk, kf);
  RowOp<BF16, D, RT> rop;
  if constexpr (BF16) {
    rop.load(reinterpret_cast<const uint16_t*>(a.q) + q_offset(a, u), a.gw, nullptr, nullptr, lane);
  } else {
    stage_rows_f32<D, RT>(a, u, q_lds, nullptr);
    __syncthreads();
    rop.bind(q_lds, lane);
  }

  // key directions: 1/|k| per key (kept in the score row for the finalize
  // kernel), then the sum of khat over the lane's keys
  const int64_t orow = out_row(a.g, u) * a.score_stride;
  float sacc[KS * 8];
#pragma unroll
  for (int i = 0; i < KS * 8; ++i) sacc[i] = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float n2 = sum_rows(kf[b].sq_norm_part());
    const float rn = n2 > 0.f ? fast_rsqrt(n2) : 0.f;   // missing keys were loaded as zeros
    const int key = key_base + (wave + 4 * b) * kBlockKeys + col;
    if (g4 == 0 && (FULL || key < u.n)) a.scores[orow + key] = rn;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) sacc[ks * 8 + e] = fmaf(rn, kf[b].at(ks, e), sacc[ks * 8 + e]);
  }

  // logits keys x rows: lane holds keys (wave + 4b)*16 + 4*g4 + i of row rt*16 + col
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 y[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) y[b] = rop.template tile<true>(kf[b], rt);
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (FULL || key_base + (wave + 4 * b) * kBlockKeys + 4 * g4 + i < u.n) mx = fmaxf(mx, y[b][i]);
    mx = xmax32(xmax16(mx));                 // max of this row over the wave's keys
    float zz = 0.f;
    if (FULL || mx != -INFINITY) {
      const float off = -mx * a.c;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (FULL || key_base + (wave + 4 * b) * kBlockKeys + 4 * g4 + i < u.n)
            zz += fast_exp2(fmaf(y[b][i], a.c, off));
    }
    zz = sum_rows(zz);
    if (g4 == 0) {
      red_m[wave][rt * 16 + col] = mx == -INFINITY ? mx : mx * a.c;
      red_z[wave][rt * 16 + col] = zz;
    }
  }
#pragma unroll
  for (int i = 0; i < KS * 8; ++i) sacc[i] = sum_in_row(sacc[i]);
  if (col == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_s[wave][32 * ks + 8 * g4 + e] = sacc[ks * 8 + e];
  }
}

// ---------------------------------------------------------------- finalize body
template <bool BF16, bool PAGED, int D, int RT, bool FULL>
__device__ __forceinline__ void finalize_body(const ScoreArgs& a, const Unit& u, int chunk,
                                              const KeyFrag<BF16, D> (&kf)[kBlocksPerWave],
                                              const RowOp<BF16, D, RT>& rop, const float* row_m,
                                              const float* row_iz) {
  constexpr int NB = kBlocksPerWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int key_base = chunk * kChunk;

  const int64_t orow = out_row(a.g, u) * a.score_stride;
  float rn[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int key = key_base + (wave + 4 * b) * kBlockKeys + col;
    rn[b] = (g4 == 0 && (FULL || key < u.n)) ? a.scores[orow + key] : 0.f;
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
  const int st0 = srow0 >> 4, st1 = srow1 >> 4;
  const float inv_nm1 = 1.f / (float)(u.n - 1);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float ip = 0.f, sd = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const bool wrows = rt * 16 < a.gw, srows = rt == st0 || rt == st1;
      if (!wrows && !srows) continue;
      const f32x4 acc = rop.template tile<false>(kf[b], rt);
      if (wrows) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ip = fmaf(fast_exp2(fmaf(acc[i], a.c, -mr[rt][i])), izr[rt][i], ip);
      }
      if (srows) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * g4 + i;
          if (r == srow0 || r == srow1) sd += acc[i];
        }
      }
    }
    ip = sum_rows(ip);
    sd = sum_rows(sd);
    const int key = key_base + (wave + 4 * b) * kBlockKeys + col;
    if (g4 == 0 && (FULL || key < u.n)) {
      const float red = rn[b] > 0.f ? (sd * rn[b] - 1.f) * inv_nm1 : 0.f;
      const float sc = a.lambda * ip - (1.f - a.lambda) * red;
      a.scores[orow + key] = sc;
      if (a.imp) a.imp[orow + key] = ip;
      if (a.red) a.red[orow + key] = red;
    }
  }
}

}  // namespace detail

using namespace detail;

// ---------------------------------------------------------------- kernel 1
template <bool BF16, bool PAGED, int D, int RT>
__global__ __launch_bounds__(kThreads) void score_stats_kernel(ScoreArgs a) {
  const int unit_id = blockIdx.x / a.max_chunks, chunk = blockIdx.x % a.max_chunks;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  const int key_base = chunk * kChunk;
  if (key_base >= u.n) return;
  if (a.reset_status) clear_status_first(a.status);
  if (a.check_blocks && step_aborted(a.status, kBadBlockId)) return;   // the pool must not be read

  __shared__ float red_m[4][RT * 16], red_z[4][RT * 16], red_s[4][D];
  __shared__ float q_lds[BF16 ? 1 : RT * 16 * D];
  if (key_base + kChunk <= u.n)
    stats_body<BF16, PAGED, D, RT, true>(a, u, unit_id, chunk, red_m, red_z, red_s, q_lds);
  else
    stats_body<BF16, PAGED, D, RT, false>(a, u, unit_id, chunk, red_m, red_z, red_s, q_lds);
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
  if (t < D) rec[2 * a.gw + t] = (red_s[0][t] + red_s[1][t]) + (red_s[2][t] + red_s[3][t]);
}

// ---------------------------------------------------------------- kernel 2
template <bool BF16, bool PAGED, int D, int RT>
__global__ __launch_bounds__(kThreads) void score_finalize_kernel(ScoreArgs a) {
  constexpr int MAXC = 8;   // records merged per batch of loads
  const int lane = threadIdx.x & (kWave - 1);
  const int item = finalize_item(blockIdx.x, gridDim.x);
  const int unit_id = item / a.max_chunks, chunk = item % a.max_chunks;
  const Unit u = decode_unit(a.g, a.tt, unit_id);
  const int key_base = chunk * kChunk;
  if (key_base >= u.n) return;
  if (a.check_blocks && step_aborted(a.status, kBadBlockId)) return;   // the pool must not be read

  __shared__ float row_m[RT * 16], row_iz[RT * 16], s_lds[D];
  __shared__ uint16_t s_bf[2][BF16 ? D : 1];
  __shared__ float q_lds[BF16 ? 1 : RT * 16 * D];

  // the chunk's keys go out first; the record merge below overlaps them
  const bool full = key_base + kChunk <= u.n;
  KeyFrag<BF16, D> kf[kBlocksPerWave];
  if (full)
    load_keys<BF16, PAGED, D, true>(a, u, chunk, kf);
  else
    load_keys<BF16, PAGED, D, false>(a, u, chunk, kf);

  // merge the unit's chunk records in a fixed order (deterministic)
  const int nch = (u.n + kChunk - 1) / kChunk;
  const float* recs = a.part + (int64_t)unit_id * a.max_chunks * a.rec;
  const int t = threadIdx.x;
  if (t < RT * 16) {
    if (t < a.gw) {
      float mm = -INFINITY, zz = 0.f;
      for (int c0 = 0; c0 < nch; c0 += MAXC) {
        float m8[MAXC], z8[MAXC];
#pragma unroll
        for (int j = 0; j < MAXC; ++j) {
          const bool ok = c0 + j < nch;
          m8[j] = ok ? recs[(c0 + j) * a.rec + t] : -INFINITY;
          z8[j] = ok ? recs[(c0 + j) * a.rec + a.gw + t] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < MAXC; ++j) merge_stats(mm, zz, m8[j], z8[j]);
      }
      row_m[t] = mm;
      row_iz[t] = 1.f / (zz * (float)a.gw);
    } else {
      row_m[t] = INFINITY;   // padding and direction-sum rows add nothing to I
      row_iz[t] = 0.f;
    }
  }
  if (t < D) {
    float sv = 0.f;
    for (int c0 = 0; c0 < nch; c0 += MAXC) {
      float s8[MAXC];
#pragma unroll
      for (int j = 0; j < MAXC; ++j) s8[j] = c0 + j < nch ? recs[(c0 + j) * a.rec + 2 * a.gw + t] : 0.f;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) sv += s8[j];
    }
    s_lds[t] = sv;
    if constexpr (BF16) {
      const uint32_t hi = f2bf_bits(sv);
      s_bf[0][t] = (uint16_t)hi;
      s_bf[1][t] = (uint16_t)f2bf_bits(sv - __uint_as_float(hi << 16));
    }
  }
  __syncthreads();

  RowOp<BF16, D, RT> rop;
  if constexpr (BF16) {
    rop.load(reinterpret_cast<const uint16_t*>(a.q) + q_offset(a, u), a.gw, s_bf[0], s_bf[1], lane);
  } else {
    stage_rows_f32<D, RT>(a, u, q_lds, s_lds);
    __syncthreads();
    rop.bind(q_lds, lane);
  }
  if (full)
    finalize_body<BF16, PAGED, D, RT, true>(a, u, chunk, kf, rop, row_m, row_iz);
  else
    finalize_body<BF16, PAGED, D, RT, false>(a, u, chunk, kf, rop, row_m, row_iz);
}

// ---------------------------------------------------------------- launch
template <bool BF16, bool PAGED, int D, int RT>
hipError_t launch_stats_t(const ScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_stats_kernel<BF16, PAGED, D, RT>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}
template <bool BF16, bool PAGED, int D, int RT>
hipError_t launch_final_t(const ScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_finalize_kernel<BF16, PAGED, D, RT>), dim3(grid), dim3(kThreads), 0, st,
                     a);
  return hipGetLastError();
}

// Both kernels of the scoring pass for one (dtype, layout, head_dim); rt1 /
// rt2 are the row tiles of the window rows and of the window + sum rows.
template <bool BF16, bool PAGED, int D>
hipError_t dispatch_score_layout(const ScoreArgs& a, int grid, int rt1, int rt2, hipStream_t st) {
  typedef hipError_t (*Fn)(const ScoreArgs&, int, hipStream_t);
#define RKV_T(F, R) F<BF16, PAGED, D, R>
  static const Fn stats[9] = {RKV_T(launch_stats_t, 1), RKV_T(launch_stats_t, 2),
                              RKV_T(launch_stats_t, 3), RKV_T(launch_stats_t, 4),
                              RKV_T(launch_stats_t, 5), RKV_T(launch_stats_t, 6),
                              RKV_T(launch_stats_t, 7), RKV_T(launch_stats_t, 8),
                              RKV_T(launch_stats_t, 9)};
  static const Fn fin[9] = {RKV_T(launch_final_t, 1), RKV_T(launch_final_t, 2),
                            RKV_T(launch_final_t, 3), RKV_T(launch_final_t, 4),
                            RKV_T(launch_final_t, 5), RKV_T(launch_final_t, 6),
                            RKV_T(launch_final_t, 7), RKV_T(launch_final_t, 8),
                            RKV_T(launch_final_t, 9)};
#undef RKV_T
  hipError_t e = stats[rt1 - 1](a, grid, st);
  if (e != hipSuccess) return e;
  return fin[rt2 - 1](a, grid, st);
}

#define RKV_DECLARE_SCORE(DT, D, L) \
  hipError_t dispatch_score_##DT##_d##D##_##L(const ScoreArgs&, int, int, int, hipStream_t);
RKV_DECLARE_SCORE(bf16, 64, contig)
RKV_DECLARE_SCORE(bf16, 64, paged)
RKV_DECLARE_SCORE(bf16, 128, contig)
RKV_DECLARE_SCORE(bf16, 128, paged)
RKV_DECLARE_SCORE(f32, 64, contig)
RKV_DECLARE_SCORE(f32, 64, paged)
RKV_DECLARE_SCORE(f32, 128, contig)
RKV_DECLARE_SCORE(f32, 128, paged)
#undef RKV_DECLARE_SCORE

}  // namespace rkv
