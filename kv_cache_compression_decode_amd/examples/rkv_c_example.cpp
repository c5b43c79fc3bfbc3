// A caller of the C ABI with no Python: builds a small bf16 KV cache with the
// HIP runtime, runs one compression step (rkv_step) and checks on the host
// what the interface promises -- lengths, keep rows (budget entries, strictly
// ascending, in range, the window at the end), compacted K/V rows equal to
// the original rows at the kept positions, sequences below the trigger left
// alone.  Prints "ok" and exits 0, or names the first failure and exits 1.
//
// Shape: 2 layers, 2 sequences (150 and 90 tokens; budget 100 + buffer 20
// triggers only the first), 4 query / 2 kv heads, head_dim 64, window 4.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "rkv.h"

namespace {

#define HIP_OK(x)                                                                 \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

// bf16 bit pattern of a float (round to nearest, ties to even)
uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// deterministic values in [-1, 1)
struct Lcg {
  uint64_t s;
  float next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) & 0xFFFFFF) / 8388608.f - 1.f;
  }
};

int fail(const char* what) {
  std::fprintf(stderr, "check failed: %s\n", what);
  return 1;
}

}  // namespace

int main() {
  const int L = 2, S = 2, HQ = 4, HKV = 2, D = 64, CAP = 160;
  const int BUDGET = 100, BUFFER = 20, WINDOW = 4;
  rkv_config cfg{};
  cfg.num_layers = L;
  cfg.num_q_heads = HQ;
  cfg.num_kv_heads = HKV;
  cfg.head_dim = D;
  cfg.budget = BUDGET;
  cfg.buffer = BUFFER;
  cfg.window = WINDOW;
  cfg.mix_lambda = 0.1f;
  cfg.dtype = RKV_DTYPE_BF16;
  cfg.layout = RKV_LAYOUT_CONTIGUOUS;
  cfg.block_size = 16;
  cfg.shared_selection = 0;
  int32_t lens[S] = {150, 90};
  const int32_t lens0[S] = {150, 90};

  const size_t kv_elems = (size_t)L * S * HKV * CAP * D;
  const size_t q_elems = (size_t)L * S * HQ * WINDOW * D;
  std::vector<uint16_t> k(kv_elems), v(kv_elems), q(q_elems);
  Lcg rng{12345};
  for (auto& x : k) x = to_bf16(rng.next());
  for (auto& x : v) x = to_bf16(rng.next());
  for (auto& x : q) x = to_bf16(rng.next());

  void *dk, *dv, *dq, *dscores, *dkeep, *dws;
  const int rows = L * S * HKV;
  const size_t ws = rkv_workspace_size(&cfg, S, CAP);
  HIP_OK(hipMalloc(&dk, kv_elems * 2));
  HIP_OK(hipMalloc(&dv, kv_elems * 2));
  HIP_OK(hipMalloc(&dq, q_elems * 2));
  HIP_OK(hipMalloc(&dscores, (size_t)rows * CAP * 4));
  HIP_OK(hipMalloc(&dkeep, (size_t)rows * BUDGET * 4));
  HIP_OK(hipMalloc(&dws, ws > 0 ? ws : 256));
  HIP_OK(hipMemcpy(dk, k.data(), kv_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v.data(), kv_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dq, q.data(), q_elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dkeep, 0xFF, (size_t)rows * BUDGET * 4));

  rkv_cache cache{};
  cache.k = dk;
  cache.v = dv;
  cache.capacity = CAP;
  int32_t free_counts[S] = {-1, -1};
  const rkv_status st = rkv_step(&cfg, &cache, dq, S, lens, (float*)dscores, CAP, (int32_t*)dkeep,
                                 nullptr, 0, free_counts, dws, ws, nullptr);
  if (st != RKV_OK) {
    std::fprintf(stderr, "rkv_step: %s (%s)\n", rkv_status_string(st), rkv_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());

  std::vector<int32_t> keep((size_t)rows * BUDGET);
  std::vector<uint16_t> k2(kv_elems), v2(kv_elems);
  HIP_OK(hipMemcpy(keep.data(), dkeep, keep.size() * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(k2.data(), dk, kv_elems * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(v2.data(), dv, kv_elems * 2, hipMemcpyDeviceToHost));

  if (lens[0] != BUDGET || lens[1] != lens0[1]) return fail("lengths after the step");
  if (free_counts[0] != 0 || free_counts[1] != 0) return fail("FREE_BLOCKS counts (contiguous: 0)");
  for (int l = 0; l < L; ++l)
    for (int s = 0; s < S; ++s)
      for (int h = 0; h < HKV; ++h) {
        const int row = (l * S + s) * HKV + h;
        const int32_t* kr = &keep[(size_t)row * BUDGET];
        const size_t base = (size_t)row * CAP * D;   // [l][s][h] rows of the cache
        if (s == 1) {   // below the trigger: keep row and cache rows untouched
          for (int i = 0; i < BUDGET; ++i)
            if (kr[i] != -1) return fail("keep row of an untriggered sequence written");
          if (std::memcmp(&k2[base], &k[base], (size_t)CAP * D * 2) != 0 ||
              std::memcmp(&v2[base], &v[base], (size_t)CAP * D * 2) != 0)
            return fail("cache of an untriggered sequence changed");
          continue;
        }
        const int n = lens0[s];
        for (int i = 0; i < BUDGET; ++i) {
          if (kr[i] < 0 || kr[i] >= n) return fail("keep entry out of range");
          if (i > 0 && kr[i] <= kr[i - 1]) return fail("keep row not strictly ascending");
          if (i >= BUDGET - WINDOW && kr[i] != n - BUDGET + i) return fail("window not kept");
          if (std::memcmp(&k2[base + (size_t)i * D], &k[base + (size_t)kr[i] * D], D * 2) != 0 ||
              std::memcmp(&v2[base + (size_t)i * D], &v[base + (size_t)kr[i] * D], D * 2) != 0)
            return fail("compacted row differs from the kept token's row");
        }
      }
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dscores));
  HIP_OK(hipFree(dkeep));
  HIP_OK(hipFree(dws));
  std::printf("ok\n");
  return 0;
}
