// Device-side helpers and launch arguments shared by the R-KV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

constexpr int kWave = 64;
constexpr int kThreads = 256;         // every kernel runs 4 waves per workgroup
constexpr int kMaxTrig = 128;         // triggered sequences per launch
constexpr int kBlockKeys = 16;        // keys per MFMA column block
constexpr int kBlocksPerWave = 4;     // column blocks a wave scores per chunk
constexpr int kChunk = kBlockKeys * kBlocksPerWave * (kThreads / kWave);  // 256 keys

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Triggered sequences of one launch, passed by value as a kernel argument.
struct TrigTable {
  int32_t seq[kMaxTrig];       // index of the sequence in the batch
  int32_t len[kMaxTrig];       // its cache length N (>= budget + buffer)
  int32_t free_off[kMaxTrig];  // paged: first FREE_BLOCKS entry of the sequence
};

// Cache geometry and method constants common to all kernels.
struct Geom {
  int32_t num_seqs, num_layers, hq, hkv, group, d, window, budget;
  int32_t paged;               // 0 contiguous, 1 paged
  int32_t cap;                 // contiguous slots per (l, s, h)
  int32_t bs_shift;            // paged: log2(block_size)
  int32_t nblk, maxblk;        // paged: pool blocks per layer, table row length
  int32_t num_trig;            // triggered sequences in this launch (device table: num_seqs)
  int32_t shared;              // 1: one keep set per (sequence, layer), from the summed scores
  int64_t layer_stride;        // elements from layer l to l + 1 of K and of V
  // Device-resident table of triggered sequences (rkv_step_device), or null
  // for the by-value TrigTable: [count][seq x num_seqs][len x num_seqs]
  // [free_off x num_seqs]; launches cover num_seqs sequences and the units of
  // table rows >= count do nothing.
  const int32_t* dtab;
};

// Workgroup barrier that orders LDS accesses only: each wave waits for its
// own LDS operations, not for its outstanding global loads -- in particular
// not for loads that stream into LDS (global_load_lds) and are waited for
// explicitly later.  The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS atomics without a return value.  Written as single instructions so
// that the compiler, which cannot tell an atomic's target apart from the
// LDS that global_load_lds is still filling, does not make them wait for
// all outstanding global loads and stores.  LDS operations complete in
// order; the next lds_barrier waits for them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_add(int* p, int v) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_min(int* p, int v) {
  asm volatile("ds_min_i32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_min(uint32_t* p, uint32_t v) {
  asm volatile("ds_min_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_max(uint32_t* p, uint32_t v) {
  asm volatile("ds_max_u32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}

// Status word flags, as in rkv.h: set on the device, read back by
// rkv_device_status.
constexpr uint32_t kSpanTimeout = RKV_DEVICE_SPAN_TIMEOUT;
constexpr uint32_t kBadBlockId = RKV_DEVICE_BAD_BLOCK_ID;

// True if a kernel of the step must leave everything untouched: the status
// word (when the call has one) holds one of the flags in mask.  Readers run
// after every kernel of the call that clears or checks the word (on the same
// stream); key-span launches, which set kSpanTimeout themselves, test only
// kBadBlockId.
__device__ __forceinline__ bool step_aborted(const uint32_t* status, uint32_t mask = ~0u) {
  return status != nullptr && (*status & mask) != 0u;
}

// Workgroup 0's first thread clears the status word (a launch that is the
// first of its call to touch it).
__device__ __forceinline__ void clear_status_first(uint32_t* status) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && status != nullptr) *status = 0u;
}

// Element offset of (layer l, kv head h)'s row 0 in a contiguous cache
// (sequence s) or in physical block 0 of a paged pool (s unused).
__device__ __forceinline__ int64_t head_base(const Geom& g, int l, int s, int h) {
  if (!g.paged) return l * g.layer_stride + (((int64_t)s * g.hkv + h) * g.cap) * g.d;
  return l * g.layer_stride + ((int64_t)h << g.bs_shift) * g.d;
}

// Units are (triggered sequence, layer, kv head), kv head fastest.
struct Unit {
  int ti, s, l, h, n;
};

// A unit whose table row is past the device table's count has n = 0: every
// kernel returns before touching memory for it.
__device__ __forceinline__ Unit decode_unit(const Geom& g, const TrigTable& tt, int u) {
  Unit r;
  r.h = u % g.hkv;
  const int lt = u / g.hkv;
  r.l = lt % g.num_layers;
  r.ti = lt / g.num_layers;
  if (g.dtab != nullptr) {
    if (r.ti >= g.dtab[0]) {
      r.s = 0;
      r.n = 0;
      return r;
    }
    r.s = g.dtab[1 + r.ti];
    r.n = g.dtab[1 + g.num_seqs + r.ti];
    return r;
  }
  r.s = tt.seq[r.ti];
  r.n = tt.len[r.ti];
  return r;
}

// First FREE_BLOCKS entry of triggered row ti.
__device__ __forceinline__ int free_off(const Geom& g, const TrigTable& tt, int ti) {
  return g.dtab != nullptr ? g.dtab[1 + 2 * g.num_seqs + ti] : tt.free_off[ti];
}

// Row index of a unit in the [L][S][Hkv][...] score / keep arrays.
__device__ __forceinline__ int64_t out_row(const Geom& g, const Unit& u) {
  return ((int64_t)u.l * g.num_seqs + u.s) * g.hkv + u.h;
}

// 16 bytes read or written once by this step (rows being compacted):
// non-temporal accesses, so the step's writes do not linger dirty in the
// caches and its single-use reads do not displace other lines.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  return make_uint4(__builtin_nontemporal_load(&p->x), __builtin_nontemporal_load(&p->y),
                    __builtin_nontemporal_load(&p->z), __builtin_nontemporal_load(&p->w));
}
__device__ __forceinline__ void stream_store(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

}  // namespace rkv
