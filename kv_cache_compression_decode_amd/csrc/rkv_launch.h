// Kernel argument blocks and host launchers of the R-KV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv_device.h"

namespace rkv {

struct ScoreArgs {
  Geom g;
  TrigTable tt;
  const void* k;          // keys (contiguous cache or paged pool)
  const void* q;          // window queries [L][S][Hq][w][d]
  const int32_t* bt;      // paged block table or nullptr
  float* scores;          // [L][S][Hkv][score_stride]
  float* imp;             // optional, same layout
  float* red;             // optional, same layout
  float* part;            // workspace: [units][max_chunks][rec] floats
  int32_t score_stride;
  int32_t max_chunks;     // chunks of the longest triggered sequence
  int32_t max_len;        // longest triggered sequence of this launch
  int32_t gw;             // window rows per unit: group * window
  int32_t rec;            // floats per chunk record: 2 * gw + d
  float lambda;
  float c;                // log2(e) / sqrt(d): raw dot -> log2-scaled logit
  // Status word of the call's workspace, or nullptr.  Key-span launches set
  // kSpanTimeout in it.  check_blocks: a prologue checked the block ids, and
  // scoring kernels return at once if it holds kBadBlockId (the pool must not
  // be read).  reset_status: this launch clears it first (the call has no
  // prologue; no earlier kernel of the call wrote it): the key-span counter
  // kernel, the single-pass kernel or the stats kernel, from workgroup 0.
  uint32_t* status;
  int32_t check_blocks;
  int32_t reset_status;
};

struct SelectArgs {
  Geom g;
  TrigTable tt;
  const float* scores;
  int32_t* keep;          // [L][S][Hkv][budget]
  int32_t score_stride;
  const uint32_t* status; // nonzero word: write nothing (nullptr: no check)
};

struct CompactArgs {
  Geom g;
  TrigTable tt;
  void* k;
  void* v;
  const int32_t* bt;
  const int32_t* keep;
  int32_t* free_blocks;   // paged FREE_BLOCKS output or nullptr
  int32_t row_bytes;      // d * element size
  const uint32_t* status; // nonzero word: touch nothing (nullptr: no check)
};

// The fused step (score + select + compact in one kernel) for units that
// fit the single-pass scoring.
struct StepArgs {
  ScoreArgs s;            // scoring arguments (keys, queries, scores, lambda, ...)
  void* k;                // keys, written by the compaction
  void* v;                // values
  int32_t* keep;          // [L][S][Hkv][budget]
  int32_t* free_blocks;   // paged FREE_BLOCKS output or nullptr
  // With s.status set: reset_status = 1 clears the word (workgroup 0; no
  // kernel before this launch in the call wrote it), else a nonzero word
  // leaves everything untouched.
  int32_t reset_status;
};

// Builds the device table of triggered sequences (Geom::dtab) from device
// lengths; sets triggered lengths to the budget and writes per-sequence
// FREE_BLOCKS counts.
struct TableArgs {
  int32_t* lens;          // device [num_seqs], in/out
  int32_t* dtab;          // device [1 + 3 * num_seqs], out
  int32_t* free_counts;   // device [num_seqs] or nullptr
  int32_t num_seqs, budget, trigger, max_len;
  int32_t block_size;     // paged block size; 0 for the contiguous layout
  uint32_t* status;       // the call's status word: cleared, then the check below
  const int32_t* bt;      // paged block table to check, or nullptr (no check)
  int32_t maxblk, nblk;   // its row length and the pool size
};

// First kernel of a call on host lengths: clears the status word (reset),
// then checks the triggered sequences' block ids against the pool (bt
// non-null) and sets kBadBlockId for an id outside [0, g.nblk).
struct PrologueArgs {
  Geom g;
  TrigTable tt;
  uint32_t* status;
  const int32_t* bt;      // paged block table to check, or nullptr
  int32_t reset;
};

// Redundancy through the explicit cosine Gram matrix (rkv_redundancy_gram).
struct GramArgs {
  Geom g;
  TrigTable tt;
  const void* k;          // keys (contiguous cache or paged pool), bf16
  const int32_t* bt;      // paged block table or nullptr
  float* red;             // [L][S][Hkv][stride]
  int32_t stride;
  int32_t units;          // triggered units of this launch (num_trig * L * Hkv)
  int32_t rows;           // rows per workgroup: gram_block_rows(longest length, d)
  int32_t rblocks;        // row blocks per unit: longest length / rows, rounded up
};

// Window-query ring store (rkv_window_store).
struct WindowArgs {
  const uint8_t* q_step;    // [count][num_seqs][hq][row_bytes]
  uint8_t* q_window;        // [L][num_seqs][hq][window][row_bytes]
  const int32_t* steps;     // device [num_seqs]: decode step of each sequence
  int32_t layer0, count, num_seqs, hq, window, row_bytes;
  int64_t pieces;           // 16-byte pieces to copy: count * num_seqs * hq * row_bytes / 16
};

hipError_t launch_window_store(const WindowArgs& a, hipStream_t st);
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st);
// Bound of the key-span wait in s_memrealtime ticks (100 MHz), process-wide.
void set_span_wait_ticks(int64_t ticks);
int64_t span_wait_ticks();
hipError_t launch_table(const TableArgs& a, hipStream_t st);
int gram_block_rows(int max_len, int d);
hipError_t launch_gram(const GramArgs& a, hipStream_t st);
hipError_t launch_score(const ScoreArgs& a, bool bf16, hipStream_t st);
// true if launch_step can run this launch's units (else use the three kernels)
bool step_fusable(const ScoreArgs& a, bool bf16);
hipError_t launch_step(const StepArgs& a, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, int max_len, hipStream_t st);
hipError_t prepare_select();   // raise the dynamic-LDS limit of the select kernel once
hipError_t launch_compact(const CompactArgs& a, hipStream_t st);

}  // namespace rkv
