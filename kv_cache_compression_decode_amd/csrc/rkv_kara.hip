// KARA-style sliding-window compression step (the KARA entry on the
// fugumt.com paper page, "KARA: Efficient Reasoning LLM Serving via
// Sliding-Window KV Cache Compression", Abstract): compress only the recently
// generated context -- the last W tokens of a sequence once W tokens have
// come since the previous compression -- scoring its tokens with
// bidirectional attention inside the window and keeping a fixed number of
// them, some widened into chunks (Token2Chunk).  Per unit (sequence, layer,
// kv head), with the G*W query rows of the G query heads that share the kv
// head and the W window keys:
//   score_j = (1 / (G W)) sum_r softmax_j(q_r . k_j / sqrt(d))   (no mask)
//   anchors = the `anchors` best tokens; each keeps every position within
//             `radius` of it (clipped to the window); the rest of the `keep`
//             places go to the best tokens outside those chunks (equal
//             scores: lower position first)
//   slots t0 .. t0+keep-1 (t0 = N - W) receive the kept tokens' K and V
//   rows in position order; the prefix [0, t0) is not touched.
//
// One 256-thread workgroup per unit does all three steps.  Every wave holds
// the W window keys in registers as MFMA operands (keys x rows products, as
// in the R-KV scoring) and takes every fourth 16-row tile of the query rows,
// so each query row is read from HBM once.  A tile's row
// softmax needs no other wave (its wave holds every key); the per-key sums
// of the weights stay in registers until the end, then one DPP row sum and
// an LDS pass over the four waves give the scores.  Query tiles reach the
// MFMA operands through a ring in LDS filled by global_load_lds, so loads of
// the next tiles are in flight without holding registers.  Selection ranks the W
// tokens by counting (W <= 128: one thread per token).  Compaction stages
// every kept row in LDS before any is written (keep[i] >= i).
// Window lengths 32, 64 and 128 are compiled.
#include "rkv_kara.h"
#include "rkv_score_impl.h"
#include "rkv_select_impl.h"

namespace rkv {

namespace {

constexpr int kKaraMaxW = 128;
constexpr int kRing = 4;   // query tiles in flight per wave

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at lds + 16 l; lds must be the same for the whole wave.
__device__ __forceinline__ void tile_piece_to_lds(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (loads retire in order: the older ones are done).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool PAGED, int D, int NB>
__global__ __launch_bounds__(kThreads) void kara_step_kernel(KaraArgs a) {
  constexpr int W = NB * kBlockKeys;
  constexpr int KS = D / 32;
  constexpr int PPR = D / 8;                          // 16-byte pieces per bf16 row
  constexpr int TILE_BYTES = 16 * D * 2;              // 16 query rows
  constexpr int NI = TILE_BYTES / (kWave * 16);       // wave-wide 16-byte loads per tile
  constexpr int WAVES = kThreads / kWave;
  static_assert(W <= kKaraMaxW, "window");
  // the compaction stages up to W rows (+ one wave's overhang) in the ring
  static_assert((W * PPR + kWave) * 16 <= (kThreads / kWave) * kRing * TILE_BYTES, "compaction buffer");
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][kRing][TILE_BYTES];
  __shared__ float part[WAVES][W];
  __shared__ __attribute__((aligned(16))) uint32_t okey[W];
  __shared__ __attribute__((aligned(16))) uint32_t okey2[W];   // 0 for tokens inside a chunk
  __shared__ int rank1[W];
  __shared__ int keep_s[W];
  __shared__ int tot[WAVES];

  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  if (u.n == 0) return;
  if (step_aborted(a.status)) return;   // a block id outside the pool: touch nothing
  const int t0 = u.n - W;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, g4 = lane >> 4;

  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
  // the W window keys: block j holds key j*16 + col, dims 32 ks + 8 g4 .. +7
  KeyFrag<true, D> kf[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) kf[j].load(a.k, rows.at(t0 + j * kBlockKeys + col), g4, true);

  // The unit's query rows, 16-row tiles; wave w takes tiles w, w + 4, ...,
  // each copied into the wave's ring of kRing tile slots, kRing - 1 tiles
  // ahead.  In a slot, piece p of row r sits at position r * PPR + (p ^ (r %
  // PPR)): the fragment reads of the 16 rows of a piece then fall on
  // different banks.
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) +
                      (((int64_t)u.l * a.g.num_seqs + u.s) * a.g.hq + (int64_t)u.h * a.g.group) * W * D;
  const int tiles = a.g.group * W / 16;
  const int my_tiles = (tiles - wave + WAVES - 1) / WAVES;   // wave-uniform
  auto issue = [&](int k) {   // tile wave + 4 k into slot k % kRing
    const int tile = wave + WAVES * k;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s = i * kWave + lane, r = s / PPR, p = (s % PPR) ^ (r % PPR);
      tile_piece_to_lds(q + (int64_t)(tile * 16 + r) * D + 8 * p, &ring[wave][k % kRing][i * kWave * 16]);
    }
  };
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k)
    if (k < my_tiles) issue(k);

  float acc[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = 0.f;
  for (int k = 0; k < my_tiles; ++k) {
    // tile k's loads are done once only the tiles issued after it are in
    // flight (min(my_tiles - 1 - k, kRing - 1) of them)
    if (k + kRing - 1 < my_tiles) issue(k + kRing - 1);
    static_assert(kRing == 4, "the waits below count up to three tiles in flight");
    switch (min(my_tiles - 1 - k, kRing - 1)) {
      case 3: wait_vm<3 * NI>(); break;
      case 2: wait_vm<2 * NI>(); break;
      case 1: wait_vm<NI>(); break;
      default: wait_vm<0>(); break;
    }
    const uint8_t* slot = ring[wave][k % kRing];
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int p = (4 * ks + g4) ^ (col % PPR);
      qf[ks] = *reinterpret_cast<const bf16x8*>(slot + (col * PPR + p) * 16);
    }
    // lane: logits of keys j*16 + 4 g4 + i against row col of the tile
    f32x4 c[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[j].w[ks]), qf[ks],
                                                       c[j], 0, 0, 0);
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, c[j][i]);
    m = xmax32(xmax16(m));           // the row's max over all W keys (raw dot; a.c > 0)
    const float off = m * a.c;       // log2 units
    float e[NB][4];
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[j][i] = fast_exp2(fmaf(c[j][i], a.c, -off));
        z += e[j][i];
      }
    const float inv = 1.f / sum_rows(z);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(e[j][i], inv, acc[j][i]);
  }
  // per key: the sum over this wave's rows (the 16 lanes of a DPP row hold
  // the 16 rows of each tile), then over the waves
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sv = sum_in_row(acc[j][i]);
      if (col == 0) part[wave][j * kBlockKeys + 4 * g4 + i] = sv;
    }
  __syncthreads();
  const int64_t orow = out_row(a.g, u);
  const float inv_rows = 1.f / (float)(a.g.group * W);
  if (t < W) {
    const float sv = ((part[0][t] + part[1][t]) + (part[2][t] + part[3][t])) * inv_rows;
    a.scores[orow * W + t] = sv;
    okey[t] = order_key(sv);
  }
  __syncthreads();

  // Token2Chunk: rank by (score desc, position asc); the `anchors` best are
  // widened to +-radius; the other places go to the best outside the chunks.
  // Ranks by counting, every thread reading all W keys (broadcast reads, four
  // at a time).  Scores are softmax means, so every order key is at least
  // 0x80000000 and a chunk token's key in okey2, 0, beats no other token.
  const int K = a.keep;
  auto count_beating = [&](const uint32_t* keys, uint32_t kt) {
    int r = 0;
#pragma unroll 8
    for (int i = 0; i < W; i += 4) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(keys + i);
      r += (k4.x > kt || (k4.x == kt && i < t)) + (k4.y > kt || (k4.y == kt && i + 1 < t)) +
           (k4.z > kt || (k4.z == kt && i + 2 < t)) + (k4.w > kt || (k4.w == kt && i + 3 < t));
    }
    return r;
  };
  const uint32_t kt = t < W ? okey[t] : 0u;
  if (t < W) rank1[t] = count_beating(okey, kt);
  __syncthreads();
  bool chunk = false;
  if (t < W) {
    for (int i = max(0, t - a.radius); i <= min(W - 1, t + a.radius); ++i) chunk |= rank1[i] < a.anchors;
    okey2[t] = chunk ? 0u : kt;
  }
  const int nchunk = __syncthreads_count(t < W && chunk);
  bool kept = chunk;
  if (t < W && !chunk) kept = count_beating(okey2, kt) < K - nchunk;
  // slot of each kept position: a workgroup scan of the flags
  const int slot = block_excl_scan<kThreads>(t < W && kept ? 1 : 0, tot);
  int32_t* krow = a.keep_out + orow * K;
  if (t < W && kept) {
    keep_s[slot] = t;
    krow[slot] = t0 + t;
  }
  __syncthreads();

  // compaction, K then V: slot t0 + i <- t0 + keep_s[i] for i < K.  The
  // kept rows are copied HBM -> LDS (the ring, idle now) with
  // global_load_lds, then written back from LDS: every row of a tensor is
  // read before any is written (keep_s[i] >= i).  Wave w takes 64-piece
  // groups w, w + 4, ...; lanes past the last piece load a kept row again
  // into the unused tail of the buffer.
  uint8_t* const stage = &ring[0][0][0];
  const int pieces = K * PPR;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    uint8_t* base = reinterpret_cast<uint8_t*>(x == 0 ? a.k : a.v);
    for (int s0 = wave * kWave; s0 < pieces; s0 += kThreads) {
      const int sp = s0 + lane, i = min(sp / PPR, K - 1), p = sp % PPR;
      tile_piece_to_lds(base + rows.at(t0 + keep_s[i]) * 2 + p * 16, stage + s0 * 16);
    }
    wait_vm<0>();
    __syncthreads();
    for (int sp = t; sp < pieces; sp += kThreads) {
      const int i = sp / PPR, p = sp % PPR;
      if (keep_s[i] != i)
        *reinterpret_cast<uint4*>(base + rows.at(t0 + i) * 2 + p * 16) =
            *reinterpret_cast<const uint4*>(stage + sp * 16);
    }
    __syncthreads();   // the buffer is read before the next tensor fills it
  }

  if (PAGED && a.free_blocks != nullptr && u.l == 0 && u.h == 0) {
    const int bs = 1 << a.g.bs_shift;
    const int first = (t0 + K + bs - 1) / bs, last = (u.n + bs - 1) / bs;
    int32_t* out = a.free_blocks + free_off(a.g, a.tt, u.ti);
    for (int b = first + t; b < last; b += kThreads) out[b - first] = a.bt[(int64_t)u.s * a.g.maxblk + b];
  }
}

template <bool PAGED, int D>
hipError_t launch_kara_t(const KaraArgs& a, int units, hipStream_t st) {
  switch (a.window_len) {
    case 32: hipLaunchKernelGGL((kara_step_kernel<PAGED, D, 2>), dim3(units), dim3(kThreads), 0, st, a); break;
    case 64: hipLaunchKernelGGL((kara_step_kernel<PAGED, D, 4>), dim3(units), dim3(kThreads), 0, st, a); break;
    case 128: hipLaunchKernelGGL((kara_step_kernel<PAGED, D, 8>), dim3(units), dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kara(const KaraArgs& a, hipStream_t st) {
  const int units = a.g.num_trig * a.g.num_layers * a.g.hkv;
  if (units == 0) return hipSuccess;
  if (a.g.d == 64) return a.g.paged ? launch_kara_t<true, 64>(a, units, st) : launch_kara_t<false, 64>(a, units, st);
  if (a.g.d == 128) return a.g.paged ? launch_kara_t<true, 128>(a, units, st) : launch_kara_t<false, 128>(a, units, st);
  return hipErrorInvalidValue;
}

}  // namespace rkv
