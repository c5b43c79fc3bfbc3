// Redundancy through the explicit cosine Gram matrix (R-KV project page on
// hysenlabs.com, "How R-KV decides what to drop"; hotdry blog post, R-KV
// section: R_j is the mean cosine similarity of key j to the unit's other
// keys, i.e. the mean off-diagonal entry of row j of the unit's N x N cosine
// matrix).
//
// One kernel.  Cosine(i, j) = (k_i . k_j) * r_i * r_j with r = 1/|k| (0 for a
// zero key), so the matrix products take the cached bf16 keys as they are
// (exact operands; no rounding of normalised keys) and the two scalings are
// applied in fp32:  R_j = (r_j * sum_i (k_j . k_i) r_i - r_j^2 |k_j|^2) / (N-1).
//
// A workgroup takes 256 or 384 rows of a unit (4 waves x 64 or 96 rows, held
// as MFMA A operands in registers; a wave whose rows all lie past N skips the
// products) and streams all of the unit's keys through LDS in
// double-buffered tiles of 64 keys (128 for the 384-row form).  Each 16 x 16 block of k_j . k_i is one chain
// of v_mfma_f32_16x16x32_bf16 (fp32 accumulation) over the head dimension;
// the row tiles' chains of one block run interleaved, and a block's
// entries are scaled by their column's r_i (while the next block's chains
// run) and summed into per-row accumulators, so the matrix never leaves
// registers (the build puts this file's MFMA results in VGPRs, where the
// scaling reads them).  The column factors r_i are computed while a tile is
// staged (the four threads loading a key reduce its squares across their
// lanes), so no pass over the keys precedes the products and no workspace is
// needed.
//
// Workgroups are mapped so that the row blocks of a unit run on one XCD
// (workgroup b runs on XCD b % 8), so a unit's later row blocks can find its
// keys in that XCD's L2; with more units in flight than an L2 holds, part of
// them come from HBM again (about 1.5 reads of every key at 1152 keys).
//
// The rank-one form in the scoring kernels gives the same values up to
// rounding with O(N d) work instead of O(N^2 d); this path computes the Gram
// formulation itself (matrix-core bound).
#include "rkv_launch.h"
#include "rkv_score_impl.h"

namespace rkv {

namespace {

constexpr int kStageKeys = kThreads / 4;   // keys staged per pass: 4 threads per key
constexpr int kWavesPerGroup = kThreads / kWave;
// Keys per LDS tile: 64, or 128 for the 96-row form at head_dim 128 (half the
// barriers per workgroup; 72 KB of LDS, two workgroups per CU as its
// registers allow anyway).
constexpr int kTile64 = 64, kTile96 = 128;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes, a native vector

// Sum of squares of the 8 bf16 values of a 16-byte piece (fp32, exact products).
__device__ __forceinline__ float sq8(const u32x4 w, float s) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xFFFF0000u);
    s = fmaf(lo, lo, fmaf(hi, hi, s));
  }
  return s;
}

// Sum over the aligned quad of lanes; every lane of the quad gets it.
__device__ __forceinline__ float sum_quad(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  return v;
}

// Staging of a tile of 64 KPT keys: thread (sk, sq) loads dims
// [QD sq, QD sq + QD) of keys sk, sk + 64, .. of tile kt (keys at or past n
// are zeros) ...
template <bool PAGED, int D, int KPT>
__device__ __forceinline__ void gram_load(u32x4 (&pre)[KPT][D / 32], const uint16_t* kc,
                                          const KeyRows<PAGED>& rows, int kt, int n, int sk, int sq) {
  constexpr int QD = D / 4, PPT = D / 32;
#pragma unroll
  for (int kk = 0; kk < KPT; ++kk) {
    const int key = (kt * KPT + kk) * kStageKeys + sk;
    const u32x4* src = reinterpret_cast<const u32x4*>(kc + rows.at(key < n ? key : 0) + QD * sq);
#pragma unroll
    for (int i = 0; i < PPT; ++i) pre[kk][i] = key < n ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
}

// ... then writes them to the LDS tile (row pitch D + 8) and, with the other
// three threads of each key, the key's 1/|k| (0 for a zero key).
template <int D, int KPT>
__device__ __forceinline__ void gram_stage(const u32x4 (&pre)[KPT][D / 32], uint16_t* tile, float* tinv, int sk,
                                           int sq) {
  constexpr int QD = D / 4, PPT = D / 32, P = D + 8;
#pragma unroll
  for (int kk = 0; kk < KPT; ++kk) {
    const int r = kk * kStageKeys + sk;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      *reinterpret_cast<u32x4*>(&tile[r * P + QD * sq + 8 * i]) = pre[kk][i];
      ss = sq8(pre[kk][i], ss);
    }
    ss = sum_quad(ss);
    if (sq == 0) tinv[r] = ss > 0.f ? fast_rsqrt(ss) : 0.f;
  }
}

// WR rows per wave (WR / 16 MFMA row tiles): each column fragment read from
// LDS feeds WR / 16 products, so more rows per wave mean less LDS traffic per
// product but more registers (at head_dim 128: 156 VGPRs and 3 waves per SIMD
// at 64 rows, 231 and 2 at 96).  TILE keys per LDS tile (a multiple of 64).
template <bool PAGED, int D, int WR, int TILE>
__global__ __launch_bounds__(kThreads) void gram_rowsum_kernel(GramArgs a) {
  constexpr int kWaveRows = WR, kRowTiles = WR / 16, kGramRows = WR * kWavesPerGroup;
  constexpr int kGramTile = TILE, KPT = TILE / kStageKeys;
  static_assert(WR % 16 == 0, "whole row tiles");
  static_assert(TILE % kStageKeys == 0, "whole staging passes per tile");
  constexpr int KS = D / 32;                             // MFMA k-steps over the head dimension
  constexpr int P = D + 8;                               // LDS row pitch (elements)
  constexpr int QD = D / 4;                              // staging: 4 threads per key, QD dims each
  constexpr int PPT = QD / 8;                            // 16-byte pieces per thread per tile
  constexpr int CT = kGramTile / 16;                     // 16-key column blocks per tile
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kGramTile * P];
  __shared__ float tinv[2][kGramTile];                  // r_i of the tile's keys
  __shared__ float nrm2[kWavesPerGroup][kWaveRows];     // |k_j|^2 of each wave's rows

  // work item of this workgroup: consecutive items (one unit's row blocks) on one XCD
  const int total = a.units * a.rblocks;
  const int per_xcd = (total + 7) / 8;
  const int w = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (w >= total) return;
  const int ui = w / a.rblocks, rb = w % a.rblocks;
  const Unit u = decode_unit(a.g, a.tt, ui);
  const int n = u.n;
  if (n == 0 || rb * kGramRows >= n) return;
  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
  const uint16_t* kc = static_cast<const uint16_t*>(a.k);
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, g4 = lane >> 4;
  const int row0 = rb * kGramRows + wave * kWaveRows;
  const bool live = row0 < n;   // wave-uniform

  // this wave's rows as A operands: row row0 + 16 rt + col, dims 32 ks + 8 g4 ..
  bf16x8 af[kRowTiles][KS];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = row0 + 16 * rt + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (r < n) v = *reinterpret_cast<const bf16x8*>(kc + rows.at(r) + 32 * ks + 8 * g4);
      af[rt][ks] = v;
    }
  }

  // staging: four threads per key
  const int sk = t >> 2, sq = t & 3;
  const int ntiles = (n + kGramTile - 1) / kGramTile;
  u32x4 pre[KPT][PPT];
  gram_load<PAGED, D, KPT>(pre, kc, rows, 0, n, sk, sq);
  gram_stage<D, KPT>(pre, &tile[0][0], tinv[0], sk, sq);
  lds_barrier();

  float racc[kRowTiles][4];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = 0.f;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) gram_load<PAGED, D, KPT>(pre, kc, rows, kt + 1, n, sk, sq);   // in flight during the products
    if (live) {
      // Block ct's four row-tile chains go into c[ct & 1] while block ct - 1's
      // results are scaled by their columns' r_i and summed into the rows.
      f32x4 c[2][kRowTiles];
      float rcol[2];
#pragma unroll
      for (int ct = 0; ct <= CT; ++ct) {
        if (ct < CT) {
          bf16x8 bf[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            bf[ks] = *reinterpret_cast<const bf16x8*>(&tile[cur][(ct * 16 + col) * P + 32 * ks + 8 * g4]);
          rcol[ct & 1] = tinv[cur][ct * 16 + col];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt)
              c[ct & 1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  af[rt][ks], bf[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : c[ct & 1][rt], 0, 0, 0);
        }
        if (ct > 0) {
          const int pb = (ct - 1) & 1;
#pragma unroll
          for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) racc[rt][i] = fmaf(c[pb][rt][i], rcol[pb], racc[rt][i]);
        }
      }
    }
    if (more) gram_stage<D, KPT>(pre, &tile[cur ^ 1][0], tinv[cur ^ 1], sk, sq);
    lds_barrier();
  }

  // |k_j|^2 of row 16 rt + col, from the A operands (4 lanes per row)
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)af[rt][ks][e];
        s = fmaf(x, x, s);
      }
    s = sum_rows(s);
    if (g4 == 0) nrm2[wave][16 * rt + col] = s;
  }
  __syncthreads();
  // lane (g4, col) holds entries of rows 4 g4 + i, column col of each 16-key block
  float* red = a.red + out_row(a.g, u) * a.stride;
  const float inv = 1.f / (float)(n - 1);
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = sum_in_row(racc[rt][i]);
      const int r = 16 * rt + 4 * g4 + i, row = row0 + r;
      const float q = nrm2[wave][r], rj = q > 0.f ? fast_rsqrt(q) : 0.f;
      if (col == 0 && row < n) red[row] = (s * rj - q * rj * rj) * inv;
    }
}

template <bool PAGED, int D, int WR, int TILE>
hipError_t launch_gram_t(const GramArgs& a, hipStream_t st) {
  const int total = a.units * a.rblocks;
  const int grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((gram_rowsum_kernel<PAGED, D, WR, TILE>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Rows per workgroup for a launch whose longest unit has max_len keys.  At
// head_dim 128 the 384-row form is taken when its last row block wastes fewer
// rows than the 256-row form's (1152 keys: 3 full blocks against 4.5); with
// equal waste, and at head_dim 64, 256 rows.
int gram_block_rows(int max_len, int d) {
  constexpr int kSmall = 64 * kWavesPerGroup, kLarge = 96 * kWavesPerGroup;
  if (d != 128) return kSmall;
  const long waste_small = (long)(max_len + kSmall - 1) / kSmall * kSmall - max_len;
  const long waste_large = (long)(max_len + kLarge - 1) / kLarge * kLarge - max_len;
  return waste_large < waste_small ? kLarge : kSmall;
}

hipError_t launch_gram(const GramArgs& a, hipStream_t st) {
  if (a.units == 0 || a.rblocks == 0) return hipSuccess;
  if (a.g.d == 64) return a.g.paged ? launch_gram_t<true, 64, 64, kTile64>(a, st) : launch_gram_t<false, 64, 64, kTile64>(a, st);
  if (a.rows == 96 * kWavesPerGroup)
    return a.g.paged ? launch_gram_t<true, 128, 96, kTile96>(a, st) : launch_gram_t<false, 128, 96, kTile96>(a, st);
  return a.g.paged ? launch_gram_t<true, 128, 64, kTile64>(a, st) : launch_gram_t<false, 128, 64, kTile64>(a, st);
}

}  // namespace rkv
