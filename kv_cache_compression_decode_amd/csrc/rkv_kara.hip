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
// in the R-KV scoring; read from one copy in LDS that the workgroup loads
// once) and takes every fourth 16-row tile of the query rows,
// so each query row is read from HBM once.  A tile's row
// softmax needs no other wave (its wave holds every key); the per-key sums
// of the weights stay in registers until the end, then one DPP row sum and
// an LDS pass over the four waves give the scores.  Query tiles reach the
// MFMA operands through a ring in LDS filled by global_load_lds, so loads of
// the next tiles are in flight without holding registers.  Selection ranks the W
// tokens by counting (W <= 128: one thread per token).  Compaction needs no
// read after the selection: the window's V rows are copied into LDS by
// global_load_lds at the start (the copies land during the scoring) and
// its K rows are the MFMA operands already in registers, so every kept row
// is written from on-chip copies (keep[i] >= i: nothing is overwritten
// before it is read).  Window lengths 32, 64 and 128 are compiled.
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

// N 16-byte LDS reads at LDS byte addresses a, a + S, .., a + (N-1) S,
// waited for inside the block.  Written as one asm block so that the
// compiler, which cannot tell these addresses apart from the LDS that
// global_load_lds copies are still filling, does not make them wait for
// every copy in flight; the caller orders them after the copies they read
// (their own s_waitcnt vmcnt and a barrier).
template <int N, int S>
__device__ __forceinline__ void lds_read_strided(uint4 (&o)[N], uint32_t a) {
  static_assert(N == 2 || N == 4 || N == 8, "2, 4 or 8 reads");
  static_assert(S % 16 == 0 && (N - 1) * S < 65536, "immediate offsets");
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:%3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1])
        : "v"(a), "i"(S)
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:%5\n\t"
        "ds_read_b128 %2, %4 offset:%6\n\t"
        "ds_read_b128 %3, %4 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a), "i"(S), "i"(2 * S), "i"(3 * S)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%9\n\t"
        "ds_read_b128 %2, %8 offset:%10\n\t"
        "ds_read_b128 %3, %8 offset:%11\n\t"
        "ds_read_b128 %4, %8 offset:%12\n\t"
        "ds_read_b128 %5, %8 offset:%13\n\t"
        "ds_read_b128 %6, %8 offset:%14\n\t"
        "ds_read_b128 %7, %8 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
          "=&v"(o[6]), "=&v"(o[7])
        : "v"(a), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S), "i"(7 * S)
        : "memory");
  }
}

// The value of lane l ^ j (j a power of two below 64; all lanes active) by
// the cheapest exchange for the distance: DPP quad permutes for 1 and 2,
// ds_swizzle's XOR mode (no LDS access) for 4 and 8, v_permlane16/32_swap
// for 16 and 32 -- whose two outputs are a lane's own value and its
// partner's, so their XOR with the own value is the partner's.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int j) {
  switch (j) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);
    case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (8 << 10) | 0x1F);
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return p[0] ^ p[1] ^ v;
    }
    default: {   // 32
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return p[0] ^ p[1] ^ v;
    }
  }
}

template <bool PAGED, int D, int NB>
__global__ __launch_bounds__(kThreads) void kara_step_kernel(KaraArgs a) {
  constexpr int W = NB * kBlockKeys;
  constexpr int KS = D / 32;
  constexpr int PPR = D / 8;                          // 16-byte pieces per bf16 row
  constexpr int TILE_BYTES = 16 * D * 2;              // 16 query rows
  constexpr int NI = TILE_BYTES / (kWave * 16);       // wave-wide 16-byte loads per tile
  constexpr int WAVES = kThreads / kWave;
  constexpr int VI = W * PPR / kThreads;              // wave-wide 16-byte loads per wave for the V rows
  static_assert(W <= kKaraMaxW, "window");
  static_assert(VI >= 1 && VI * kThreads == W * PPR, "V rows in whole wave-wide loads");
  // The window's K rows go through LDS (once per workgroup) unless that
  // would cost the CU its second workgroup (LDS bytes: ring, V rows, K rows,
  // and the small arrays below); else every wave loads them itself.
  constexpr int kRowsLds = W * PPR * 16;
  constexpr int kOtherLds = WAVES * kRing * TILE_BYTES + kRowsLds + 44 * W + 8 * WAVES;
  constexpr bool KLDS = kOtherLds + kRowsLds <= 80 * 1024 || kOtherLds > 80 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][kRing][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vwin[W * PPR * 16];   // the window's V rows
  __shared__ __attribute__((aligned(16))) uint8_t kwin[KLDS ? kRowsLds : 16];   // its K rows (swizzled)
  __shared__ float part[WAVES][W];
  __shared__ __attribute__((aligned(16))) uint32_t okey[W];
  __shared__ uint64_t xchg[W];   // bitonic exchange across the two waves
  __shared__ int rank1[W];
  __shared__ int kflag[W];
  __shared__ int keep_s[W];
  __shared__ int slot_of[W];
  __shared__ int tot[WAVES], tot2[WAVES];

  const Unit u = decode_unit(a.g, a.tt, blockIdx.x);
  if (u.n == 0) return;
  if (step_aborted(a.status)) return;   // a block id outside the pool: touch nothing
  const int t0 = u.n - W;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int col = lane & 15, g4 = lane >> 4;

  KeyRows<PAGED> rows;
  rows.init(a.g, a.bt, u);
  // the window's K rows into LDS once per workgroup (every wave needs all of
  // them; loading them per wave spends the CU's load bandwidth four times):
  // piece p of row r at position r * PPR + (p ^ (r % PPR)), so that the
  // fragment reads below fall on different banks; the oldest loads of every
  // wave.  (Without room for that copy, each wave loads the keys into its
  // registers.)
  const uint8_t* const ksrc = reinterpret_cast<const uint8_t*>(a.k);
  KeyFrag<true, D> kf[NB];
  if constexpr (KLDS) {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int s0 = (wave * VI + i) * kWave, sp = s0 + lane, r = sp / PPR, p = (sp % PPR) ^ (r % PPR);
      tile_piece_to_lds(ksrc + rows.at(t0 + r) * 2 + p * 16, kwin + s0 * 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) kf[j].load(a.k, rows.at(t0 + j * kBlockKeys + col), g4, true);
  }

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
  // the window's V rows into LDS (piece p of row r at r * PPR + p); used by
  // the compaction only, so issued after the first tile's products (before
  // the loop in a wave without tiles), out of the start-up stream that the
  // first products wait for
  uint8_t* const vbase = reinterpret_cast<uint8_t*>(a.v);
  auto issue_v = [&] {
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int s0 = (wave * VI + i) * kWave, sp = s0 + lane;
      tile_piece_to_lds(vbase + rows.at(t0 + sp / PPR) * 2 + (sp % PPR) * 16, vwin + s0 * 16);
    }
  };
  if (my_tiles == 0) issue_v();
  // Loads retire in order: wait until only the n latest tiles (and, if v,
  // the V rows issued after the first tiles) are in flight.
  static_assert(kRing == 4, "the waits count up to three tiles in flight");
  auto wait_tiles = [&](int n, bool v) {
    if (v) {
      switch (n) {
        case 3: wait_vm<3 * NI + VI>(); break;
        case 2: wait_vm<2 * NI + VI>(); break;
        case 1: wait_vm<NI + VI>(); break;
        default: wait_vm<VI>(); break;
      }
    } else {
      switch (n) {
        case 3: wait_vm<3 * NI>(); break;
        case 2: wait_vm<2 * NI>(); break;
        case 1: wait_vm<NI>(); break;
        default: wait_vm<0>(); break;
      }
    }
  };

  // K rows in LDS for every wave (the first tiles and the V rows may still
  // be in flight); then the W window keys as MFMA operands: block j holds
  // key j*16 + col, dims 32 ks + 8 g4 .. +7
  if constexpr (KLDS) {
    wait_tiles(min(my_tiles, kRing - 1), my_tiles == 0);
    lds_barrier();
    // one read block per 32-dim slice: piece 4 ks + g4 of key j*16 + col sits
    // at (j*16 + col) * PPR + ((4 ks + g4) ^ col) -- key block j a constant
    // 16 rows further than block 0 (r % PPR = col for every block)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 o[NB];
      lds_read_strided<NB, kBlockKeys * PPR * 16>(
          o, lds_addr(kwin + (col * PPR + ((4 * ks + g4) ^ (col % PPR))) * 16));
#pragma unroll
      for (int j = 0; j < NB; ++j) kf[j].w[ks] = o[j];
    }
  }

  float acc[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = 0.f;
  for (int k = 0; k < my_tiles; ++k) {
    // tile k's loads are done once only the tiles issued after it are in
    // flight (min(my_tiles - 1 - k, kRing - 1) of them), and the V rows if
    // they were issued after it (at the end of iteration 0, after tiles
    // 0 .. min(kRing, my_tiles) - 1)
    if (k + kRing - 1 < my_tiles) issue(k + kRing - 1);
    wait_tiles(min(my_tiles - 1 - k, kRing - 1), k >= 1 && k < min(kRing, my_tiles));
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
    if (k == 0) issue_v();
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
  // A bitonic sort of the W composite keys (order key, then 255 - position:
  // unique, larger is better), one per thread of the first W, exchanges
  // across lanes (partner distance < 64, lane_xor) or through LDS (64).  Sorted index
  // = rank.  The fill takes the first K - |chunks| non-chunk tokens in that
  // order (a scan over the sorted positions).
  const int K = a.keep;
  uint64_t ck = t < W ? ((uint64_t)okey[t] << 8) | (uint64_t)(255 - t) : 0ull;
#pragma unroll
  for (int kk = 2; kk <= W; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      uint64_t other;
      if (j < kWave) {
        const uint32_t lo = lane_xor((uint32_t)ck, j);
        const uint32_t hi = lane_xor((uint32_t)(ck >> 32), j);
        other = ((uint64_t)hi << 32) | lo;
      } else {
        __syncthreads();
        if (t < W) xchg[t] = ck;
        __syncthreads();
        other = t < W ? xchg[t ^ j] : 0ull;
      }
      // descending within blocks of kk whose index bit kk is clear
      const bool desc = (t & kk) == 0, lower = (t & j) == 0;
      const uint64_t hi_v = ck > other ? ck : other, lo_v = ck > other ? other : ck;
      ck = (desc == lower) ? hi_v : lo_v;
    }
  }
  const int spos = 255 - (int)(ck & 0xFFu);   // token at sorted index t (t < W)
  if (t < W) rank1[spos] = t;
  __syncthreads();
  bool chunk = false;
  if (t < W) {
    for (int i = max(0, t - a.radius); i <= min(W - 1, t + a.radius); ++i) chunk |= rank1[i] < a.anchors;
    kflag[t] = chunk ? 1 : 0;
  }
  const int nchunk = __syncthreads_count(t < W && chunk);
  // in sorted order: the first K - nchunk tokens outside the chunks
  const bool sorted_free = t < W && kflag[spos] == 0;
  const int before = block_excl_scan<kThreads>(sorted_free ? 1 : 0, tot2);
  if (sorted_free && before < K - nchunk) kflag[spos] = 1;
  __syncthreads();
  const bool kept = t < W && kflag[t] != 0;
  // slot of each kept position: a workgroup scan of the flags
  const int slot = block_excl_scan<kThreads>(kept ? 1 : 0, tot);
  int32_t* krow = a.keep_out + orow * K;
  if (t < W) slot_of[t] = kept ? slot : -1;
  if (t < W && kept) {
    keep_s[slot] = t;
    krow[slot] = t0 + t;
  }
  wait_vm<0>();      // this wave's V rows are in LDS
  __syncthreads();   // slots, and every wave's V rows

  // compaction: row t0 + i <- row t0 + keep_s[i] for i < K, rows that move
  // only.  K from the registers: wave w writes key blocks w, w + 4, ...
  // (lane (col, g4) holds pieces 4 ks + g4 of key 16 j + col).  V from LDS.
  uint8_t* const kbase = reinterpret_cast<uint8_t*>(a.k);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (j % WAVES != wave) continue;
    const int s = j * kBlockKeys + col, sl = slot_of[s];
    if (sl >= 0 && sl != s) {
      uint8_t* dst = kbase + rows.at(t0 + sl) * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<uint4*>(dst + (4 * ks + g4) * 16) = kf[j].w[ks];
    }
  }
  for (int sp = t; sp < K * PPR; sp += kThreads) {
    const int i = sp / PPR, p = sp % PPR, src = keep_s[i];
    if (src != i)
      *reinterpret_cast<uint4*>(vbase + rows.at(t0 + i) * 2 + p * 16) =
          *reinterpret_cast<const uint4*>(vwin + (src * PPR + p) * 16);
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
