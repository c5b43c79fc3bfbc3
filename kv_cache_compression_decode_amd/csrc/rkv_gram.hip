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
// A workgroup takes 128 rows of a unit (4 waves x 32 rows, held as MFMA A
// operands in registers) and streams all of the unit's keys through LDS in
// double-buffered 64-key tiles.  Each 16 x 16 block of k_j . k_i is one chain
// of v_mfma_f32_16x16x32_bf16 (fp32 accumulation) over the head dimension;
// its entries are scaled by their column's r_i and summed into per-row
// accumulators, so the matrix never leaves registers.  The column factors
// r_i are computed while a tile is staged (the threads loading a key reduce
// its squares across their lanes), so no pass over the keys precedes the
// products and no workspace is needed.
//
// Workgroups are mapped so that the row blocks of a unit run on one XCD
// (workgroup b runs on XCD b % 8): the unit's keys are read from HBM into
// that XCD's L2 once and re-read from there by its other row blocks.
//
// The rank-one form in the scoring kernels gives the same values up to
// rounding with O(N d) work instead of O(N^2 d); this path computes the Gram
// formulation itself (matrix-core bound).
#include "rkv_launch.h"
#include "rkv_score_impl.h"

namespace rkv {

namespace {

constexpr int kGramRows = 128;   // rows per workgroup: 4 waves x 32
constexpr int kGramTile = 64;    // keys per LDS tile
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes, a native vector

// Sum over aligned groups of G consecutive lanes (G = 8 or 16); every lane of
// the group gets it.
template <int G>
__device__ __forceinline__ float sum_lanes(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
  if (G == 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float sq8(const u32x4 w) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xFFFF0000u);
    s = fmaf(lo, lo, fmaf(hi, hi, s));
  }
  return s;
}

template <bool PAGED, int D>
__global__ __launch_bounds__(kThreads) void gram_rowsum_kernel(GramArgs a) {
  constexpr int KS = D / 32;                             // MFMA k-steps over the head dimension
  constexpr int P = D + 8;                               // LDS row pitch (elements)
  constexpr int TPK = D / 8;                             // threads per key when staging
  constexpr int PPT = kGramTile * TPK / kThreads;        // 16-byte pieces per thread per tile
  static_assert(kGramTile * TPK % kThreads == 0, "tile pieces spread evenly");
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kGramTile * P];
  __shared__ float tinv[2][kGramTile];                  // r_i of the tile's keys
  __shared__ float nrm2[kThreads / kWave][32];          // |k_j|^2 of each wave's rows

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
  const int row0 = rb * kGramRows + wave * 32;

  // this wave's 32 rows as A operands: row row0 + 16 rt + col, dims 32 ks + 8 g4 ..
  bf16x8 af[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = row0 + 16 * rt + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 v = {};
      if (r < n) v = *reinterpret_cast<const bf16x8*>(kc + rows.at(r) + 32 * ks + 8 * g4);
      af[rt][ks] = v;
    }
  }

  // Tile loads: piece pc = t + i * kThreads is key pc / TPK of the tile, dims
  // 8 (pc % TPK) ..; keys at or past n are zeros.
  const int ntiles = (n + kGramTile - 1) / kGramTile;
  u32x4 pre[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int pc = t + i * kThreads, key = pc / TPK;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < n) v = *reinterpret_cast<const u32x4*>(kc + rows.at(key) + 8 * (pc % TPK));
    pre[i] = v;
  }
  // staged keys into LDS buffer b, with their column factors
#define GRAM_STAGE(b)                                                                          \
  _Pragma("unroll") for (int i = 0; i < PPT; ++i) {                                            \
    const int pc = t + i * kThreads, key = pc / TPK;                                           \
    *reinterpret_cast<u32x4*>(&tile[b][key * P + 8 * (pc % TPK)]) = pre[i];                    \
    const float s = sum_lanes<TPK>(sq8(pre[i]));                                               \
    if (pc % TPK == 0) tinv[b][key] = s > 0.f ? fast_rsqrt(s) : 0.f;                           \
  }
  GRAM_STAGE(0)
  lds_barrier();

  float racc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) racc[rt][i] = 0.f;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) {   // the next tile's loads in flight during this tile's products
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = t + i * kThreads, key = (kt + 1) * kGramTile + pc / TPK;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < n) v = *reinterpret_cast<const u32x4*>(kc + rows.at(key) + 8 * (pc % TPK));
        pre[i] = v;
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      bf16x8 bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bf[ks] = *reinterpret_cast<const bf16x8*>(&tile[cur][(ct * 16 + col) * P + 32 * ks + 8 * g4]);
      const float ri = tinv[cur][ct * 16 + col];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][ks], bf[ks], c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) racc[rt][i] = fmaf(c[i], ri, racc[rt][i]);
      }
    }
    if (more) GRAM_STAGE(cur ^ 1)
    lds_barrier();
  }
#undef GRAM_STAGE

  // |k_j|^2 of row 16 rt + col, from the A operands (4 lanes per row)
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
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
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s = sum_in_row(racc[rt][i]);
      const int r = 16 * rt + 4 * g4 + i, row = row0 + r;
      const float q = nrm2[wave][r], rj = q > 0.f ? fast_rsqrt(q) : 0.f;
      if (col == 0 && row < n) red[row] = (s * rj - q * rj * rj) * inv;
    }
}

template <bool PAGED, int D>
hipError_t launch_gram_t(const GramArgs& a, hipStream_t st) {
  const int total = a.units * a.rblocks;
  const int grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((gram_rowsum_kernel<PAGED, D>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int gram_row_blocks(int max_len) { return (max_len + kGramRows - 1) / kGramRows; }

hipError_t launch_gram(const GramArgs& a, hipStream_t st) {
  if (a.units == 0 || a.rblocks == 0) return hipSuccess;
  if (a.g.d == 64) return a.g.paged ? launch_gram_t<true, 64>(a, st) : launch_gram_t<false, 64>(a, st);
  return a.g.paged ? launch_gram_t<true, 128>(a, st) : launch_gram_t<false, 128>(a, st);
}

}  // namespace rkv
