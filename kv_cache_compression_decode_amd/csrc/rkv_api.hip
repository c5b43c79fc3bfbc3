// Host side of the C ABI declared in include/rkv.h: argument checks, the
// table of triggered sequences, workspace sizing and kernel launches.
// Every check runs before anything is enqueued; errors are returned with a
// thread-local detail message and never thrown across the interface.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "rkv.h"
#include "rkv_kara.h"
#include "rkv_launch.h"

namespace {

thread_local std::string g_err;

rkv_status fail(rkv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

rkv_status hip_fail(hipError_t e, const char* what) {
  return fail(RKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Every workspace starts with this many bytes holding the status word.
constexpr size_t kStatusBytes = 256;

uint32_t* status_of(void* ws) { return static_cast<uint32_t*>(ws); }
float* records_of(void* ws) {
  return reinterpret_cast<float*>(static_cast<char*>(ws) + kStatusBytes);
}

int ilog2_exact(int v) {
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// The model and cache shape of a config (every entry point).
rkv_status check_shape(const rkv_config* c) {
  if (c == nullptr) return fail(RKV_ERR_INVALID_ARG, "cfg is NULL");
  if (c->num_layers < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1)
    return fail(RKV_ERR_INVALID_ARG, "num_layers, num_q_heads and num_kv_heads must be >= 1");
  if (c->num_q_heads % c->num_kv_heads != 0)
    return fail(RKV_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                c->num_q_heads, c->num_kv_heads);
  if (c->dtype != RKV_DTYPE_F32 && c->dtype != RKV_DTYPE_BF16)
    return fail(RKV_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (c->layout != RKV_LAYOUT_CONTIGUOUS && c->layout != RKV_LAYOUT_PAGED)
    return fail(RKV_ERR_INVALID_ARG, "unknown layout %d", c->layout);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(RKV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  if (c->layout == RKV_LAYOUT_PAGED) {
    if (c->block_size < 1) return fail(RKV_ERR_INVALID_ARG, "block_size must be >= 1");
    if (ilog2_exact(c->block_size) < 0 || c->block_size > 1024)
      return fail(RKV_ERR_UNSUPPORTED, "block_size %d (supported: powers of two up to 1024)",
                  c->block_size);
  }
  if (c->check_block_table != 0 && c->check_block_table != 1)
    return fail(RKV_ERR_INVALID_ARG, "check_block_table must be 0 or 1");
  return RKV_OK;
}

rkv_status check_config(const rkv_config* c) {
  rkv_status st = check_shape(c);
  if (st != RKV_OK) return st;
  if (c->window < 1) return fail(RKV_ERR_INVALID_ARG, "window must be >= 1");
  if (c->budget <= c->window)
    return fail(RKV_ERR_INVALID_ARG, "budget (%d) must exceed window (%d)", c->budget, c->window);
  if (c->buffer < 1) return fail(RKV_ERR_INVALID_ARG, "buffer must be >= 1");
  if (!(c->mix_lambda >= 0.f && c->mix_lambda <= 1.f))
    return fail(RKV_ERR_INVALID_ARG, "mix_lambda must lie in [0, 1]");
  const long gw = (long)(c->num_q_heads / c->num_kv_heads) * c->window;
  if (gw > RKV_MAX_WINDOW_ROWS)
    return fail(RKV_ERR_UNSUPPORTED, "group * window = %ld exceeds %d", gw, RKV_MAX_WINDOW_ROWS);
  if (c->budget > RKV_MAX_LEN)
    return fail(RKV_ERR_UNSUPPORTED, "budget %d exceeds %d", c->budget, RKV_MAX_LEN);
  if (c->shared_selection != 0 && c->shared_selection != 1)
    return fail(RKV_ERR_INVALID_ARG, "shared_selection must be 0 or 1");
  return RKV_OK;
}

// True if the call checks block ids on the device (paged layout only).
bool checks_blocks(const rkv_config* c) {
  return c->layout == RKV_LAYOUT_PAGED && c->check_block_table == 1;
}

// Elements of one layer of K (or V) when packed.
int64_t packed_layer(const rkv_config* c, const rkv_cache* k, int32_t num_seqs) {
  if (c->layout == RKV_LAYOUT_CONTIGUOUS)
    return (int64_t)num_seqs * c->num_kv_heads * k->capacity * c->head_dim;
  return (int64_t)k->num_blocks * c->num_kv_heads * c->block_size * c->head_dim;
}

rkv_status check_cache(const rkv_config* c, const rkv_cache* k, bool need_v, int32_t num_seqs) {
  if (k == nullptr) return fail(RKV_ERR_INVALID_ARG, "cache is NULL");
  if (k->k == nullptr) return fail(RKV_ERR_INVALID_ARG, "cache->k is NULL");
  if (need_v && k->v == nullptr) return fail(RKV_ERR_INVALID_ARG, "cache->v is NULL");
  if (!aligned16(k->k) || (need_v && !aligned16(k->v)))
    return fail(RKV_ERR_INVALID_ARG, "cache->k / cache->v must be 16-byte aligned");
  if (c->layout == RKV_LAYOUT_CONTIGUOUS) {
    if (k->capacity < 1) return fail(RKV_ERR_INVALID_ARG, "capacity must be >= 1");
  } else {
    if (k->num_blocks < 1) return fail(RKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
    if (k->block_table == nullptr) return fail(RKV_ERR_INVALID_ARG, "block_table is NULL");
    if (k->max_blocks_per_seq < 1) return fail(RKV_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  }
  if (k->layer_stride < 0) return fail(RKV_ERR_INVALID_ARG, "layer_stride must be >= 0");
  const int64_t esize = c->dtype == RKV_DTYPE_BF16 ? 2 : 4;
  if (k->layer_stride != 0 && (k->layer_stride * esize) % 16 != 0)
    return fail(RKV_ERR_INVALID_ARG, "layer_stride of %lld elements is not a multiple of 16 bytes",
                (long long)k->layer_stride);
  const int64_t packed = packed_layer(c, k, num_seqs < 0 ? 0 : num_seqs);
  if (k->layer_stride != 0 && c->num_layers > 1 && k->layer_stride < packed)
    return fail(RKV_ERR_INVALID_ARG, "layer_stride %lld is below the %lld elements of one layer",
                (long long)k->layer_stride, (long long)packed);
  return RKV_OK;
}

struct Trig {
  int32_t seq, len;
};

// Triggered sequences, with length checks against the cache geometry.
// `cache` may be NULL (selection needs no geometry).
rkv_status collect(const rkv_config* c, const rkv_cache* cache, int32_t num_seqs,
                   const int32_t* lens, std::vector<Trig>& out) {
  out.clear();
  if (num_seqs < 0) return fail(RKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs > 0 && lens == nullptr) return fail(RKV_ERR_INVALID_ARG, "h_seq_lens is NULL");
  const long trigger = (long)c->budget + c->buffer;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = lens[s];
    if (n < 0) return fail(RKV_ERR_INVALID_ARG, "h_seq_lens[%d] = %d is negative", s, n);
    if (n < trigger) continue;
    if (n > RKV_MAX_LEN)
      return fail(RKV_ERR_UNSUPPORTED, "h_seq_lens[%d] = %d exceeds %d", s, n, RKV_MAX_LEN);
    if (cache != nullptr) {
      if (c->layout == RKV_LAYOUT_CONTIGUOUS && n > cache->capacity)
        return fail(RKV_ERR_INVALID_ARG, "h_seq_lens[%d] = %d exceeds capacity %d", s, n,
                    cache->capacity);
      if (c->layout == RKV_LAYOUT_PAGED && (long)n > (long)cache->max_blocks_per_seq * c->block_size)
        return fail(RKV_ERR_INVALID_ARG, "h_seq_lens[%d] = %d exceeds the block table (%d blocks)",
                    s, n, cache->max_blocks_per_seq);
    }
    out.push_back({s, n});
  }
  return RKV_OK;
}

rkv::Geom make_geom(const rkv_config* c, const rkv_cache* cache, int32_t num_seqs) {
  rkv::Geom g{};
  g.num_seqs = num_seqs;
  g.num_layers = c->num_layers;
  g.hq = c->num_q_heads;
  g.hkv = c->num_kv_heads;
  g.group = c->num_q_heads / c->num_kv_heads;
  g.d = c->head_dim;
  g.window = c->window;
  g.budget = c->budget;
  g.paged = c->layout == RKV_LAYOUT_PAGED;
  if (cache != nullptr) {
    g.cap = cache->capacity;
    g.nblk = cache->num_blocks;
    g.maxblk = cache->max_blocks_per_seq;
    g.layer_stride = cache->layer_stride != 0 ? cache->layer_stride : packed_layer(c, cache, num_seqs);
  }
  g.bs_shift = g.paged ? ilog2_exact(c->block_size) : 0;
  g.shared = c->shared_selection;
  return g;
}

// Fill the triggered table for trig[first, first + count).
void fill_table(rkv::TrigTable& tt, const std::vector<Trig>& trig, size_t first, int count,
                const int32_t* free_off) {
  for (int i = 0; i < count; ++i) {
    tt.seq[i] = trig[first + i].seq;
    tt.len[i] = trig[first + i].len;
    tt.free_off[i] = free_off ? free_off[first + i] : 0;
  }
}

int32_t max_len_of(const std::vector<Trig>& trig, size_t first, size_t count) {
  int32_t m = 0;
  for (size_t i = first; i < first + count; ++i) m = std::max(m, trig[i].len);
  return m;
}

size_t record_floats(const rkv_config* c) {
  return 2 * (size_t)(c->num_q_heads / c->num_kv_heads) * c->window + c->head_dim;
}

size_t ws_bytes_for(const rkv_config* c, long seqs, long max_len) {
  const long t = std::min<long>(seqs, rkv::kMaxTrig);
  const long chunks = (max_len + rkv::kChunk - 1) / rkv::kChunk;
  const size_t bytes = (size_t)t * c->num_layers * c->num_kv_heads * chunks * record_floats(c) * 4;
  return kStatusBytes + ((bytes + 255) & ~(size_t)255);
}

rkv::ScoreArgs make_score_args(const rkv_config* cfg, const rkv_cache* cache, const void* q,
                               int32_t num_seqs, float* scores, int32_t score_stride,
                               float* imp, float* red, void* workspace) {
  rkv::ScoreArgs a{};
  a.g = make_geom(cfg, cache, num_seqs);
  a.k = cache->k;
  a.q = q;
  a.bt = cache->block_table;
  a.scores = scores;
  a.imp = imp;
  a.red = red;
  a.part = workspace != nullptr ? records_of(workspace) : nullptr;
  a.status = workspace != nullptr ? status_of(workspace) : nullptr;
  a.score_stride = score_stride;
  a.gw = a.g.group * cfg->window;
  a.rec = (int32_t)record_floats(cfg);
  a.lambda = cfg->mix_lambda;
  a.c = (float)(1.4426950408889634 / sqrt((double)cfg->head_dim));
  return a;
}

// FREE_BLOCKS counts (closed form) and per-triggered-sequence offsets.
rkv_status free_block_plan(const rkv_config* cfg, int32_t num_seqs, const std::vector<Trig>& trig,
                           int32_t* free_blocks, int32_t free_capacity,
                           std::vector<int32_t>& counts, std::vector<int32_t>& offs) {
  counts.assign(num_seqs > 0 ? num_seqs : 0, 0);
  offs.assign(trig.size(), 0);
  if (cfg->layout != RKV_LAYOUT_PAGED) return RKV_OK;
  const int bs = cfg->block_size;
  const long kept_blocks = ((long)cfg->budget + bs - 1) / bs;
  long total = 0;
  for (size_t i = 0; i < trig.size(); ++i) {
    const long used = ((long)trig[i].len + bs - 1) / bs;
    const int32_t c = (int32_t)std::max(0L, used - kept_blocks);
    counts[trig[i].seq] = c;
    offs[i] = (int32_t)total;
    total += c;
  }
  if (total > 0 && free_blocks == nullptr) return fail(RKV_ERR_INVALID_ARG, "free_blocks is NULL");
  if (total > free_capacity)
    return fail(RKV_ERR_INVALID_ARG, "free_capacity %d below the %ld freed blocks", free_capacity,
                total);
  return RKV_OK;
}

// Device path (rkv_step_device): the status word, then the table, then the
// scoring records.
size_t dev_table_bytes(long seqs) { return ((size_t)(1 + 3 * seqs) * 4 + 255) & ~(size_t)255; }

size_t dev_records_bytes(const rkv_config* c, long seqs, long max_len) {
  const long chunks = (max_len + rkv::kChunk - 1) / rkv::kChunk;
  const size_t b = (size_t)seqs * c->num_layers * c->num_kv_heads * chunks * record_floats(c) * 4;
  return (b + 255) & ~(size_t)255;
}

bool dev_fusable(const rkv_config* c, int32_t max_len) {
  rkv::ScoreArgs a{};
  a.g.d = c->head_dim;
  a.g.shared = c->shared_selection;
  a.gw = (c->num_q_heads / c->num_kv_heads) * c->window;
  a.max_len = max_len;
  return rkv::step_fusable(a, c->dtype == RKV_DTYPE_BF16);
}

}  // namespace


namespace {

rkv_status check_ws(const void* ws, size_t bytes, size_t need) {
  if (ws == nullptr) return fail(RKV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned256(ws)) return fail(RKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < need) return fail(RKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", bytes, need);
  return RKV_OK;
}

// The prologue of one launch's triggered rows: clear the status word
// (reset), check their block ids (check).
hipError_t prologue(const rkv::Geom& g, const rkv::TrigTable& tt, void* ws, const rkv_cache* cache,
                    bool reset, bool check, hipStream_t hs) {
  rkv::PrologueArgs p{};
  p.g = g;
  p.tt = tt;
  p.status = status_of(ws);
  p.bt = check ? cache->block_table : nullptr;
  p.reset = reset ? 1 : 0;
  return rkv::launch_prologue(p, hs);
}

// rkv_step (also behind the allocation-free entry point).  Launches of at
// most kMaxTrig sequences each; those that cannot run fused score, then
// select, then compact -- scoring of all of them first, so that a device
// check failing in any of them stops every write of the call -- and the
// fused launches come last.  The status word is cleared by the call's first
// kernel that touches it: the block-check prologue, else the first scoring
// launch, else the first fused launch.
rkv_status step_impl(const rkv_config* cfg, const rkv_cache* cache, const void* q_window,
                     int32_t num_seqs, int32_t* h_seq_lens, float* scores, int32_t score_stride,
                     int32_t* keep, int32_t* free_blocks, int32_t free_capacity,
                     int32_t* h_free_counts, void* workspace, size_t workspace_bytes,
                     hipStream_t hs) {
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  std::vector<Trig> trig;
  if ((st = check_cache(cfg, cache, true, num_seqs)) != RKV_OK) return st;
  if ((st = collect(cfg, cache, num_seqs, h_seq_lens, trig)) != RKV_OK) return st;
  std::vector<int32_t> counts, offs;
  if ((st = free_block_plan(cfg, num_seqs, trig, free_blocks, free_capacity, counts, offs)) != RKV_OK)
    return st;
  const bool bf16 = cfg->dtype == RKV_DTYPE_BF16;
  const bool paged = cfg->layout == RKV_LAYOUT_PAGED;
  const bool check = checks_blocks(cfg);
  if (!trig.empty()) {
    if (q_window == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_window is NULL");
    if (!aligned16(q_window)) return fail(RKV_ERR_INVALID_ARG, "q_window must be 16-byte aligned");
    if (scores == nullptr) return fail(RKV_ERR_INVALID_ARG, "scores is NULL");
    if (keep == nullptr) return fail(RKV_ERR_INVALID_ARG, "keep is NULL");
    const int32_t maxn = max_len_of(trig, 0, trig.size());
    if (score_stride < maxn)
      return fail(RKV_ERR_INVALID_ARG, "score_stride %d is below the longest triggered length %d",
                  score_stride, maxn);
    rkv::ScoreArgs a = make_score_args(cfg, cache, q_window, num_seqs, scores, score_stride,
                                       nullptr, nullptr, workspace);
    struct Launch {
      size_t first;
      int cnt, max_len;
      bool fused;
    };
    std::vector<Launch> plan;
    bool any_unfused = false;
    for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
      const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
      a.max_len = max_len_of(trig, first, cnt);
      const bool fused = rkv::step_fusable(a, bf16);
      plan.push_back({first, cnt, a.max_len, fused});
      if (fused) continue;
      any_unfused = true;
      // launches that cannot run fused need the scoring workspace
      if ((st = check_ws(workspace, workspace_bytes, ws_bytes_for(cfg, cnt, a.max_len))) != RKV_OK)
        return st;
    }
    if (check && workspace == nullptr)
      return fail(RKV_ERR_WORKSPACE, "check_block_table needs a workspace");
    if (workspace != nullptr && (st = check_ws(workspace, workspace_bytes, kStatusBytes)) != RKV_OK)
      return st;
    {
      const hipError_t e = rkv::prepare_select();
      if (e != hipSuccess) return hip_fail(e, "select kernel LDS limit");
    }
    hipError_t e;
    if (check) {
      for (size_t i = 0; i < plan.size(); ++i) {
        fill_table(a.tt, trig, plan[i].first, plan[i].cnt, nullptr);
        a.g.num_trig = plan[i].cnt;
        if ((e = prologue(a.g, a.tt, workspace, cache, i == 0, true, hs)) != hipSuccess)
          return hip_fail(e, "prologue launch");
      }
    }
    a.check_blocks = check ? 1 : 0;
    bool reset_pending = workspace != nullptr && !check;
    auto set_launch = [&](const Launch& p) {
      fill_table(a.tt, trig, p.first, p.cnt, offs.data());
      a.g.num_trig = p.cnt;
      a.max_len = p.max_len;
      a.max_chunks = (a.max_len + rkv::kChunk - 1) / rkv::kChunk;
    };
    for (const Launch& p : plan) {
      if (p.fused) continue;
      set_launch(p);
      a.reset_status = reset_pending ? 1 : 0;
      reset_pending = false;
      if ((e = rkv::launch_score(a, bf16, hs)) != hipSuccess) return hip_fail(e, "score launch");
    }
    a.reset_status = 0;
    for (const Launch& p : plan) {
      if (p.fused) continue;
      set_launch(p);
      rkv::SelectArgs sl{};
      sl.g = a.g;
      sl.tt = a.tt;
      sl.scores = scores;
      sl.keep = keep;
      sl.score_stride = score_stride;
      sl.status = a.status;
      if ((e = rkv::launch_select(sl, a.max_len, hs)) != hipSuccess) return hip_fail(e, "select launch");
    }
    for (const Launch& p : plan) {
      if (p.fused) continue;
      set_launch(p);
      rkv::CompactArgs ca{};
      ca.g = a.g;
      ca.tt = a.tt;
      ca.k = cache->k;
      ca.v = cache->v;
      ca.bt = cache->block_table;
      ca.keep = keep;
      ca.free_blocks = paged ? free_blocks : nullptr;
      ca.row_bytes = cfg->head_dim * (bf16 ? 2 : 4);
      ca.status = a.status;
      if ((e = rkv::launch_compact(ca, hs)) != hipSuccess) return hip_fail(e, "compact launch");
    }
    // fused launches: after a kernel of the call touched the status word
    // they check it; else the first of them clears it
    const bool touched = check || any_unfused;
    for (const Launch& p : plan) {
      if (!p.fused) continue;
      set_launch(p);
      rkv::StepArgs sa{};
      sa.s = a;
      sa.s.status = touched || reset_pending ? status_of(workspace) : nullptr;
      sa.reset_status = reset_pending ? 1 : 0;
      reset_pending = false;
      sa.k = cache->k;
      sa.v = cache->v;
      sa.keep = keep;
      sa.free_blocks = paged ? free_blocks : nullptr;
      if ((e = rkv::launch_step(sa, hs)) != hipSuccess) return hip_fail(e, "step launch");
    }
  }
  for (const Trig& t : trig) h_seq_lens[t.seq] = cfg->budget;
  if (h_free_counts != nullptr)
    for (int32_t s = 0; s < num_seqs; ++s) h_free_counts[s] = counts[s];
  return RKV_OK;
}

// Scratch of the allocation-free entry point: the workspace rkv_step would
// take, in a device array of the library's own (each GPU holds its copy at
// its own address until the process ends).  Host code never passes the
// array's name to a kernel or a copy: only the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kScratchBytes = (size_t)32 << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
rkv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RKV_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned256(p)) return fail(RKV_ERR_HIP, "scratch has no usable address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RKV_OK;
}

}  // namespace

extern "C" {

const char* rkv_status_string(rkv_status s) {
  switch (s) {
    case RKV_OK: return "RKV_OK";
    case RKV_ERR_INVALID_ARG: return "RKV_ERR_INVALID_ARG";
    case RKV_ERR_UNSUPPORTED: return "RKV_ERR_UNSUPPORTED";
    case RKV_ERR_WORKSPACE: return "RKV_ERR_WORKSPACE";
    case RKV_ERR_HIP: return "RKV_ERR_HIP";
    case RKV_ERR_DEVICE_CHECK: return "RKV_ERR_DEVICE_CHECK";
  }
  return "RKV_ERR_UNKNOWN";
}

const char* rkv_last_error(void) { return g_err.c_str(); }

int32_t rkv_is_triggered(const rkv_config* cfg, int32_t len) {
  if (cfg == nullptr) return -1;
  return (long)len >= (long)cfg->budget + cfg->buffer ? 1 : 0;
}

size_t rkv_workspace_size(const rkv_config* cfg, int32_t num_seqs, int32_t max_len) {
  if (check_config(cfg) != RKV_OK || num_seqs < 0 || max_len < 0) return 0;
  return ws_bytes_for(cfg, num_seqs, max_len);
}

rkv_status rkv_score(const rkv_config* cfg, const rkv_cache* cache, const void* q_window,
                     int32_t num_seqs, const int32_t* h_seq_lens, float* scores,
                     int32_t score_stride, float* importance, float* redundancy, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  std::vector<Trig> trig;
  if ((st = check_cache(cfg, cache, false, num_seqs)) != RKV_OK) return st;
  if ((st = collect(cfg, cache, num_seqs, h_seq_lens, trig)) != RKV_OK) return st;
  if (trig.empty()) return RKV_OK;
  if (q_window == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_window is NULL");
  if (!aligned16(q_window)) return fail(RKV_ERR_INVALID_ARG, "q_window must be 16-byte aligned");
  if (scores == nullptr) return fail(RKV_ERR_INVALID_ARG, "scores is NULL");
  const int32_t maxn = max_len_of(trig, 0, trig.size());
  if (score_stride < maxn)
    return fail(RKV_ERR_INVALID_ARG, "score_stride %d is below the longest triggered length %d",
                score_stride, maxn);
  for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
    const size_t cnt = std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
    const size_t need = ws_bytes_for(cfg, (long)cnt, max_len_of(trig, first, cnt));
    if ((st = check_ws(workspace, workspace_bytes, need)) != RKV_OK) return st;
  }

  rkv::ScoreArgs a = make_score_args(cfg, cache, q_window, num_seqs, scores, score_stride,
                                     importance, redundancy, workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool check = checks_blocks(cfg);
  a.check_blocks = check ? 1 : 0;
  for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
    const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
    fill_table(a.tt, trig, first, cnt, nullptr);
    a.g.num_trig = cnt;
    a.max_len = max_len_of(trig, first, cnt);
    a.max_chunks = (a.max_len + rkv::kChunk - 1) / rkv::kChunk;
    hipError_t e;
    // the status word: cleared (and the block ids checked) by a prologue when
    // checking, else cleared by the first scoring launch itself
    if (check && (e = prologue(a.g, a.tt, workspace, cache, first == 0, true, hs)) != hipSuccess)
      return hip_fail(e, "prologue launch");
    a.reset_status = !check && first == 0 ? 1 : 0;
    e = rkv::launch_score(a, cfg->dtype == RKV_DTYPE_BF16, hs);
    if (e != hipSuccess) return hip_fail(e, "score launch");
  }
  return RKV_OK;
}

rkv_status rkv_window_store(const rkv_config* cfg, int32_t layer0, int32_t layer_count,
                            const void* q_step, int32_t num_seqs, const int32_t* d_steps,
                            void* q_window, void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  if (num_seqs < 0) return fail(RKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (layer0 < 0 || layer_count < 0 || (int64_t)layer0 + layer_count > cfg->num_layers)
    return fail(RKV_ERR_INVALID_ARG, "layers [%d, %d + %d) are outside [0, %d)", layer0, layer0,
                layer_count, cfg->num_layers);
  if (num_seqs == 0 || layer_count == 0) return RKV_OK;
  if (q_step == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_step is NULL");
  if (d_steps == nullptr) return fail(RKV_ERR_INVALID_ARG, "d_steps is NULL");
  if (q_window == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_window is NULL");
  if (!aligned16(q_step) || !aligned16(q_window))
    return fail(RKV_ERR_INVALID_ARG, "q_step and q_window must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(d_steps) & 3u) != 0)
    return fail(RKV_ERR_INVALID_ARG, "d_steps must be 4-byte aligned");
  rkv::WindowArgs a{};
  a.q_step = static_cast<const uint8_t*>(q_step);
  a.q_window = static_cast<uint8_t*>(q_window);
  a.steps = d_steps;
  a.layer0 = layer0;
  a.count = layer_count;
  a.num_seqs = num_seqs;
  a.hq = cfg->num_q_heads;
  a.window = cfg->window;
  a.row_bytes = cfg->head_dim * (cfg->dtype == RKV_DTYPE_BF16 ? 2 : 4);
  a.pieces = (int64_t)layer_count * num_seqs * cfg->num_q_heads * (a.row_bytes / 16);
  const hipError_t e = rkv::launch_window_store(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "window store launch");
  return RKV_OK;
}

rkv_status rkv_redundancy_gram(const rkv_config* cfg, const rkv_cache* cache, int32_t num_seqs,
                               const int32_t* h_seq_lens, float* redundancy, int32_t stride,
                               void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  if (cfg->dtype != RKV_DTYPE_BF16)
    return fail(RKV_ERR_UNSUPPORTED, "rkv_redundancy_gram takes bf16 caches");
  std::vector<Trig> trig;
  if ((st = check_cache(cfg, cache, false, num_seqs)) != RKV_OK) return st;
  if ((st = collect(cfg, cache, num_seqs, h_seq_lens, trig)) != RKV_OK) return st;
  if (trig.empty()) return RKV_OK;
  if (redundancy == nullptr) return fail(RKV_ERR_INVALID_ARG, "redundancy is NULL");
  const int32_t maxn = max_len_of(trig, 0, trig.size());
  if (stride < maxn)
    return fail(RKV_ERR_INVALID_ARG, "stride %d is below the longest triggered length %d", stride,
                maxn);
  rkv::GramArgs a{};
  a.g = make_geom(cfg, cache, num_seqs);
  a.k = cache->k;
  a.bt = cache->block_table;
  a.red = redundancy;
  a.stride = stride;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
    const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
    fill_table(a.tt, trig, first, cnt, nullptr);
    a.g.num_trig = cnt;
    a.units = cnt * cfg->num_layers * cfg->num_kv_heads;
    const int longest = max_len_of(trig, first, cnt);
    a.rows = rkv::gram_block_rows(longest, cfg->head_dim);
    a.rblocks = (longest + a.rows - 1) / a.rows;
    const hipError_t e = rkv::launch_gram(a, hs);
    if (e != hipSuccess) return hip_fail(e, "gram launch");
  }
  return RKV_OK;
}

rkv_status rkv_select(const rkv_config* cfg, int32_t num_seqs, const int32_t* h_seq_lens,
                      const float* scores, int32_t score_stride, int32_t* keep, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  std::vector<Trig> trig;
  if ((st = collect(cfg, nullptr, num_seqs, h_seq_lens, trig)) != RKV_OK) return st;
  if (trig.empty()) return RKV_OK;
  if (scores == nullptr) return fail(RKV_ERR_INVALID_ARG, "scores is NULL");
  if (keep == nullptr) return fail(RKV_ERR_INVALID_ARG, "keep is NULL");
  const int32_t maxn = max_len_of(trig, 0, trig.size());
  if (score_stride < maxn)
    return fail(RKV_ERR_INVALID_ARG, "score_stride %d is below the longest triggered length %d",
                score_stride, maxn);
  if (workspace != nullptr && (st = check_ws(workspace, workspace_bytes, kStatusBytes)) != RKV_OK)
    return st;
  {
    hipError_t e = rkv::prepare_select();
    if (e != hipSuccess) return hip_fail(e, "select kernel LDS limit");
  }
  rkv::SelectArgs a{};
  a.g = make_geom(cfg, nullptr, num_seqs);
  a.scores = scores;
  a.keep = keep;
  a.score_stride = score_stride;
  a.status = workspace != nullptr ? status_of(workspace) : nullptr;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
    const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
    fill_table(a.tt, trig, first, cnt, nullptr);
    a.g.num_trig = cnt;
    hipError_t e = rkv::launch_select(a, max_len_of(trig, first, cnt), hs);
    if (e != hipSuccess) return hip_fail(e, "select launch");
  }
  return RKV_OK;
}

rkv_status rkv_compact(const rkv_config* cfg, const rkv_cache* cache, int32_t num_seqs,
                       int32_t* h_seq_lens, const int32_t* keep, int32_t* free_blocks,
                       int32_t free_capacity, int32_t* h_free_counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  std::vector<Trig> trig;
  if ((st = check_cache(cfg, cache, true, num_seqs)) != RKV_OK) return st;
  if ((st = collect(cfg, cache, num_seqs, h_seq_lens, trig)) != RKV_OK) return st;
  const bool paged = cfg->layout == RKV_LAYOUT_PAGED;
  const bool check = checks_blocks(cfg);
  std::vector<int32_t> counts, offs;
  if ((st = free_block_plan(cfg, num_seqs, trig, free_blocks, free_capacity, counts, offs)) != RKV_OK)
    return st;
  if (!trig.empty() && keep == nullptr) return fail(RKV_ERR_INVALID_ARG, "keep is NULL");
  if (!trig.empty() && check && workspace == nullptr)
    return fail(RKV_ERR_WORKSPACE, "check_block_table needs a workspace");
  if (workspace != nullptr && (st = check_ws(workspace, workspace_bytes, kStatusBytes)) != RKV_OK)
    return st;
  if (!trig.empty()) {
    rkv::CompactArgs a{};
    a.g = make_geom(cfg, cache, num_seqs);
    a.k = cache->k;
    a.v = cache->v;
    a.bt = cache->block_table;
    a.keep = keep;
    a.free_blocks = paged ? free_blocks : nullptr;
    a.row_bytes = cfg->head_dim * (cfg->dtype == RKV_DTYPE_BF16 ? 2 : 4);
    a.status = workspace != nullptr ? status_of(workspace) : nullptr;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
      const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
      fill_table(a.tt, trig, first, cnt, offs.data());
      a.g.num_trig = cnt;
      hipError_t e;
      if (check && (e = prologue(a.g, a.tt, workspace, cache, false, true, hs)) != hipSuccess)
        return hip_fail(e, "prologue launch");
      e = rkv::launch_compact(a, hs);
      if (e != hipSuccess) return hip_fail(e, "compact launch");
    }
  }
  for (const Trig& t : trig) h_seq_lens[t.seq] = cfg->budget;
  if (h_free_counts != nullptr)
    for (int32_t s = 0; s < num_seqs; ++s) h_free_counts[s] = counts[s];
  return RKV_OK;
}

rkv_status rkv_step(const rkv_config* cfg, const rkv_cache* cache, const void* q_window,
                    int32_t num_seqs, int32_t* h_seq_lens, float* scores, int32_t score_stride,
                    int32_t* keep, int32_t* free_blocks, int32_t free_capacity,
                    int32_t* h_free_counts, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return step_impl(cfg, cache, q_window, num_seqs, h_seq_lens, scores, score_stride, keep,
                   free_blocks, free_capacity, h_free_counts, workspace, workspace_bytes,
                   static_cast<hipStream_t>(stream));
}

size_t rkv_step_device_workspace_size(const rkv_config* cfg, int32_t num_seqs, int32_t max_len) {
  if (check_config(cfg) != RKV_OK || num_seqs < 0 || max_len < 0 || max_len > RKV_MAX_LEN) return 0;
  size_t b = kStatusBytes + dev_table_bytes(num_seqs);
  if (!dev_fusable(cfg, max_len)) b += dev_records_bytes(cfg, num_seqs, max_len);
  return b;
}

rkv_status rkv_step_device(const rkv_config* cfg, const rkv_cache* cache, const void* q_window,
                           int32_t num_seqs, int32_t* d_seq_lens, int32_t max_len, float* scores,
                           int32_t score_stride, int32_t* keep, int32_t* free_blocks,
                           int32_t free_capacity, int32_t* d_free_counts, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err.clear();
  rkv_status st = check_config(cfg);
  if (st != RKV_OK) return st;
  if ((st = check_cache(cfg, cache, true, num_seqs)) != RKV_OK) return st;
  if (num_seqs < 0) return fail(RKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return RKV_OK;
  if (d_seq_lens == nullptr) return fail(RKV_ERR_INVALID_ARG, "d_seq_lens is NULL");
  if (max_len < 0) return fail(RKV_ERR_INVALID_ARG, "max_len must be >= 0");
  if (max_len > RKV_MAX_LEN)
    return fail(RKV_ERR_UNSUPPORTED, "max_len %d exceeds %d", max_len, RKV_MAX_LEN);
  const bool paged = cfg->layout == RKV_LAYOUT_PAGED;
  const bool bf16 = cfg->dtype == RKV_DTYPE_BF16;
  if (!paged && max_len > cache->capacity)
    return fail(RKV_ERR_INVALID_ARG, "max_len %d exceeds capacity %d", max_len, cache->capacity);
  if (paged && (long)max_len > (long)cache->max_blocks_per_seq * cfg->block_size)
    return fail(RKV_ERR_INVALID_ARG, "max_len %d exceeds the block table (%d blocks)", max_len,
                cache->max_blocks_per_seq);
  if (q_window == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_window is NULL");
  if (!aligned16(q_window)) return fail(RKV_ERR_INVALID_ARG, "q_window must be 16-byte aligned");
  if (scores == nullptr) return fail(RKV_ERR_INVALID_ARG, "scores is NULL");
  if (keep == nullptr) return fail(RKV_ERR_INVALID_ARG, "keep is NULL");
  if (score_stride < max_len)
    return fail(RKV_ERR_INVALID_ARG, "score_stride %d is below max_len %d", score_stride, max_len);
  if (paged) {
    const long bs = cfg->block_size;
    const long per = std::max(0L, (max_len + bs - 1) / bs - (cfg->budget + bs - 1) / bs);
    const long need = per * num_seqs;
    if (need > 0 && free_blocks == nullptr) return fail(RKV_ERR_INVALID_ARG, "free_blocks is NULL");
    if (need > free_capacity)
      return fail(RKV_ERR_INVALID_ARG, "free_capacity %d below the %ld entries of the worst case",
                  free_capacity, need);
  }
  if ((st = check_ws(workspace, workspace_bytes,
                     rkv_step_device_workspace_size(cfg, num_seqs, max_len))) != RKV_OK)
    return st;
  {
    const hipError_t e = rkv::prepare_select();
    if (e != hipSuccess) return hip_fail(e, "select kernel LDS limit");
  }

  int32_t* dtab = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kStatusBytes);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  rkv::TableArgs ta{};
  ta.lens = d_seq_lens;
  ta.dtab = dtab;
  ta.free_counts = d_free_counts;
  ta.num_seqs = num_seqs;
  ta.budget = cfg->budget;
  ta.trigger = cfg->budget + cfg->buffer;
  ta.max_len = max_len;
  ta.block_size = paged ? cfg->block_size : 0;
  ta.status = status_of(workspace);
  ta.bt = checks_blocks(cfg) ? cache->block_table : nullptr;
  ta.maxblk = cache->max_blocks_per_seq;
  ta.nblk = cache->num_blocks;
  hipError_t e = rkv::launch_table(ta, hs);
  if (e != hipSuccess) return hip_fail(e, "table launch");
  if (max_len < (long)cfg->budget + cfg->buffer) return RKV_OK;   // nothing can trigger

  rkv::ScoreArgs a = make_score_args(cfg, cache, q_window, num_seqs, scores, score_stride,
                                     nullptr, nullptr, workspace);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(dtab) + dev_table_bytes(num_seqs));
  a.g.num_trig = num_seqs;
  a.g.dtab = dtab;
  a.check_blocks = checks_blocks(cfg) ? 1 : 0;   // the table kernel cleared and checked it
  a.max_len = max_len;
  a.max_chunks = (max_len + rkv::kChunk - 1) / rkv::kChunk;
  if (rkv::step_fusable(a, bf16)) {
    rkv::StepArgs sa{};
    sa.s = a;   // status checked: the table kernel cleared and set it
    sa.k = cache->k;
    sa.v = cache->v;
    sa.keep = keep;
    sa.free_blocks = paged ? free_blocks : nullptr;
    e = rkv::launch_step(sa, hs);
    if (e != hipSuccess) return hip_fail(e, "step launch");
    return RKV_OK;
  }
  e = rkv::launch_score(a, bf16, hs);
  if (e != hipSuccess) return hip_fail(e, "score launch");
  rkv::SelectArgs sl{};
  sl.g = a.g;
  sl.scores = scores;
  sl.keep = keep;
  sl.score_stride = score_stride;
  sl.status = a.status;
  e = rkv::launch_select(sl, max_len, hs);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  rkv::CompactArgs ca{};
  ca.g = a.g;
  ca.k = cache->k;
  ca.v = cache->v;
  ca.bt = cache->block_table;
  ca.keep = keep;
  ca.free_blocks = paged ? free_blocks : nullptr;
  ca.row_bytes = cfg->head_dim * (bf16 ? 2 : 4);
  ca.status = a.status;
  e = rkv::launch_compact(ca, hs);
  if (e != hipSuccess) return hip_fail(e, "compact launch");
  return RKV_OK;
}

rkv_status rkv_step_noalloc(const rkv_config* cfg, const rkv_cache* cache, const void* q_window,
                            int32_t num_seqs, int32_t* h_seq_lens, float* scores,
                            int32_t score_stride, int32_t* keep, int32_t* free_blocks,
                            int32_t free_capacity, int32_t* h_free_counts, void* stream) {
  g_err.clear();
  void* ws = nullptr;
  rkv_status st = scratch_address(&ws);
  if (st != RKV_OK) return st;
  st = step_impl(cfg, cache, q_window, num_seqs, h_seq_lens, scores, score_stride, keep,
                 free_blocks, free_capacity, h_free_counts, ws, kScratchBytes,
                 static_cast<hipStream_t>(stream));
  if (st == RKV_ERR_WORKSPACE)
    return fail(RKV_ERR_WORKSPACE, "the step needs more scratch than the %zu bytes rkv_step_noalloc holds (%s)",
                kScratchBytes, g_err.c_str());
  return st;
}

rkv_status rkv_kara_step(const rkv_config* cfg, const rkv_kara_config* kc, const rkv_cache* cache,
                         const void* q_tail, int32_t num_seqs, int32_t* h_seq_lens,
                         int32_t* h_tail_start, float* scores, int32_t* keep, int32_t* free_blocks,
                         int32_t free_capacity, int32_t* h_free_counts, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err.clear();
  rkv_status st = check_shape(cfg);
  if (st != RKV_OK) return st;
  if (cfg->dtype != RKV_DTYPE_BF16) return fail(RKV_ERR_UNSUPPORTED, "rkv_kara_step takes bf16 caches");
  if (kc == nullptr) return fail(RKV_ERR_INVALID_ARG, "kara config is NULL");
  const int W = kc->window_len, K = kc->keep;
  if (W != 32 && W != 64 && W != 128)
    return fail(RKV_ERR_UNSUPPORTED, "window_len %d (supported: 32, 64, 128)", W);
  if (K < 1 || K > W) return fail(RKV_ERR_INVALID_ARG, "keep %d outside [1, window_len %d]", K, W);
  if (kc->anchors < 0 || kc->radius < 0)
    return fail(RKV_ERR_INVALID_ARG, "anchors and radius must be >= 0");
  if ((long)kc->anchors * (2L * kc->radius + 1) > K)
    return fail(RKV_ERR_INVALID_ARG, "anchors * (2 radius + 1) = %ld exceeds keep %d",
                (long)kc->anchors * (2L * kc->radius + 1), K);
  if ((st = check_cache(cfg, cache, true, num_seqs)) != RKV_OK) return st;
  if (num_seqs < 0) return fail(RKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs > 0 && (h_seq_lens == nullptr || h_tail_start == nullptr))
    return fail(RKV_ERR_INVALID_ARG, "h_seq_lens and h_tail_start must not be NULL");
  const bool paged = cfg->layout == RKV_LAYOUT_PAGED;
  const bool check = checks_blocks(cfg);
  std::vector<Trig> trig;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = h_seq_lens[s], tail = h_tail_start[s];
    if (n < 0 || tail < 0 || tail > n)
      return fail(RKV_ERR_INVALID_ARG, "sequence %d: length %d, tail start %d", s, n, tail);
    if ((long)n - tail < W) continue;
    if (n > RKV_MAX_LEN) return fail(RKV_ERR_UNSUPPORTED, "h_seq_lens[%d] = %d exceeds %d", s, n, RKV_MAX_LEN);
    if (!paged && n > cache->capacity)
      return fail(RKV_ERR_INVALID_ARG, "h_seq_lens[%d] = %d exceeds capacity %d", s, n, cache->capacity);
    if (paged && (long)n > (long)cache->max_blocks_per_seq * cfg->block_size)
      return fail(RKV_ERR_INVALID_ARG, "h_seq_lens[%d] = %d exceeds the block table (%d blocks)", s, n,
                  cache->max_blocks_per_seq);
    trig.push_back({s, n});
  }
  std::vector<int32_t> counts(num_seqs > 0 ? num_seqs : 0, 0), offs(trig.size(), 0);
  long total = 0;
  if (paged) {
    const long bs = cfg->block_size;
    for (size_t i = 0; i < trig.size(); ++i) {
      const long n = trig[i].len, n_new = n - W + K;
      counts[trig[i].seq] = (int32_t)((n + bs - 1) / bs - (n_new + bs - 1) / bs);
      offs[i] = (int32_t)total;
      total += counts[trig[i].seq];
    }
    if (total > 0 && free_blocks == nullptr) return fail(RKV_ERR_INVALID_ARG, "free_blocks is NULL");
    if (total > free_capacity)
      return fail(RKV_ERR_INVALID_ARG, "free_capacity %d below the %ld freed blocks", free_capacity, total);
  }
  if (!trig.empty()) {
    if (q_tail == nullptr) return fail(RKV_ERR_INVALID_ARG, "q_tail is NULL");
    if (!aligned16(q_tail)) return fail(RKV_ERR_INVALID_ARG, "q_tail must be 16-byte aligned");
    if (scores == nullptr || keep == nullptr) return fail(RKV_ERR_INVALID_ARG, "scores and keep must not be NULL");
    if (check && workspace == nullptr) return fail(RKV_ERR_WORKSPACE, "check_block_table needs a workspace");
    if (workspace != nullptr && (st = check_ws(workspace, workspace_bytes, kStatusBytes)) != RKV_OK)
      return st;
    rkv::KaraArgs a{};
    a.g = make_geom(cfg, cache, num_seqs);
    a.q = q_tail;
    a.k = cache->k;
    a.v = cache->v;
    a.bt = cache->block_table;
    a.scores = scores;
    a.keep_out = keep;
    a.free_blocks = paged ? free_blocks : nullptr;
    a.status = check ? status_of(workspace) : nullptr;
    a.window_len = W;
    a.keep = K;
    a.anchors = kc->anchors;
    a.radius = kc->radius;
    a.c = (float)(1.4426950408889634 / sqrt((double)cfg->head_dim));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    for (size_t first = 0; first < trig.size(); first += rkv::kMaxTrig) {
      const int cnt = (int)std::min<size_t>(rkv::kMaxTrig, trig.size() - first);
      fill_table(a.tt, trig, first, cnt, offs.data());
      a.g.num_trig = cnt;
      hipError_t e;
      if (check && (e = prologue(a.g, a.tt, workspace, cache, first == 0, true, hs)) != hipSuccess)
        return hip_fail(e, "prologue launch");
      if ((e = rkv::launch_kara(a, hs)) != hipSuccess) return hip_fail(e, "kara launch");
    }
  }
  for (const Trig& t : trig) {
    h_seq_lens[t.seq] = t.len - W + K;
    h_tail_start[t.seq] = t.len - W + K;
  }
  if (h_free_counts != nullptr)
    for (int32_t s = 0; s < num_seqs; ++s) h_free_counts[s] = counts[s];
  return RKV_OK;
}

rkv_status rkv_device_status(const void* workspace, void* stream, uint32_t* flags) {
  g_err.clear();
  if (workspace == nullptr) {   // the allocation-free entry's scratch
    void* ws = nullptr;
    const rkv_status st = scratch_address(&ws);
    if (st != RKV_OK) return st;
    workspace = ws;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e, "status read");
  if (flags != nullptr) *flags = word;
  if (word == 0) return RKV_OK;
  return fail(RKV_ERR_DEVICE_CHECK, "device check failed (flags 0x%x:%s%s); the cache was left as it was",
              word, (word & RKV_DEVICE_SPAN_TIMEOUT) ? " key-span wait timed out" : "",
              (word & RKV_DEVICE_BAD_BLOCK_ID) ? " block id outside the pool" : "");
}

int64_t rkv_set_span_wait_us(int64_t microseconds) {
  if (microseconds < 0 || microseconds > 60000000) return -1;
  const int64_t prev = rkv::span_wait_ticks() / 100;
  rkv::set_span_wait_ticks(microseconds * 100);   // s_memrealtime: 100 MHz
  return prev;
}

}  // extern "C"
