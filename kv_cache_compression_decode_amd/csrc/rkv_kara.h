// Arguments and launcher of the KARA-style window step (rkv_kara.hip).
#pragma once

#include "rkv_launch.h"

namespace rkv {

// KARA-style window step (rkv_kara_step): score the last window_len tokens
// of each triggered unit with bidirectional attention, keep `keep` of them
// (Token2Chunk), compact them after the prefix.
struct KaraArgs {
  Geom g;
  TrigTable tt;
  const void* q;          // window-token queries [L][S][Hq][window_len][d]
  void* k;                // keys (contiguous cache or paged pool), bf16
  void* v;                // values
  const int32_t* bt;      // paged block table or nullptr
  float* scores;          // [L][S][Hkv][window_len]
  int32_t* keep_out;      // [L][S][Hkv][keep], absolute positions
  int32_t* free_blocks;   // paged FREE_BLOCKS output or nullptr
  const uint32_t* status; // nonzero word: touch nothing (nullptr: no check)
  int32_t window_len, keep, anchors, radius;
  float c;                // log2(e) / sqrt(d)
};

hipError_t launch_kara(const KaraArgs& a, hipStream_t st);

}  // namespace rkv
