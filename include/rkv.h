/*
 * rkv.h -- C ABI of the R-KV decode-time KV-cache compression step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step (R-KV project page on hysenlabs.com, "R-KV: Redundancy-Aware KV
 * Cache Compression for Reasoning Models", section "How R-KV decides what to
 * drop: budget, buffer and cross-layer scoring"; hotdry blog post on R-KV /
 * EvolKV / Ada-KV, R-KV section) runs for every sequence whose cache has
 * reached budget + buffer tokens.  For each triggered (sequence, layer, kv
 * head) -- a "unit" -- it
 *   1. scores each cached token j:
 *        importance  I_j = mean over the window queries of the query heads
 *                          that share the kv head of softmax_j(q . k_j / sqrt(d))
 *                          (softmax over all N cached keys),
 *        redundancy  R_j = mean cosine similarity of k_j to the other N-1 keys,
 *        score       S_j = lambda * I_j - (1 - lambda) * R_j;
 *   2. keeps the last `window` tokens and the best budget - window of the
 *      others (larger S first, equal S: lower position first);
 *   3. compacts K and V in place so that slot i holds the i-th kept token in
 *      position order; the sequence then holds `budget` tokens, and in the
 *      paged layout the emptied blocks are reported (FREE_BLOCKS).
 *
 * Conventions for every call
 *   - Device pointers are caller-owned; the library never allocates, frees or
 *     keeps them.  Host pointers are read (and, where stated, written) during
 *     the call only.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous: results are valid once the stream reaches that point.
 *   - bf16 units longer than one workgroup holds (more than 1280 keys at
 *     head_dim 128, 2560 at 64) are scored by several workgroups that wait
 *     for one another (rkv_score, and rkv_step / rkv_step_device when they
 *     fall back to the three kernels).  A workgroup takes its span from a
 *     ticket it draws when it starts, so a span only waits for spans that
 *     started before it or that the next starting workgroups take, and one
 *     such launch always completes; two of them running at the same time on
 *     different streams of one device can hold each other's room: run such
 *     calls on one stream (or one at a time).  The
 *     wait is bounded (one second by default, rkv_set_span_wait_us), so the
 *     device never hangs.  A wait that reaches the bound sets
 *     RKV_DEVICE_SPAN_TIMEOUT in the workspace's status word; selection and
 *     compaction given that workspace then leave the keep rows and the cache
 *     untouched, and rkv_device_status reports it.
 *   - Every argument is checked before anything is enqueued.  On an error the
 *     call returns a status other than RKV_OK, enqueues nothing and changes no
 *     output; rkv_last_error() then describes it.  No C++ exception crosses
 *     this interface.  A device fault of earlier work shows up as RKV_ERR_HIP.
 *   - Checks that need device data (a key-span wait that timed out, a block
 *     id outside the pool) are recorded in the status word at the start of
 *     the workspace (see rkv_device_status): the calls given that workspace
 *     then skip every later write of the step, so the cache keeps its input
 *     contents.
 *   - Sequence lengths live on the host.  Sequences below the trigger are
 *     untouched: their cache rows, score rows and keep rows are not written.
 *   - A call covers all layers and all triggered sequences of the batch.
 *
 * Layouts (row-major, element = the cache dtype unless stated)
 *   contiguous K, V : [num_layers][num_seqs][num_kv_heads][capacity][head_dim]
 *   paged K, V pool : [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 *                     token t of sequence s lives in physical block
 *                     block_table[s * max_blocks_per_seq + t / block_size],
 *                     row t % block_size; every layer uses the same table.
 *                     Block ids must lie in [0, num_blocks): they are checked
 *                     only with cfg->check_block_table = 1 (below).
 *   layer stride    : cache->layer_stride elements from layer l to layer l + 1
 *                     of K (and of V); 0 means the packed layouts above.
 *   window queries  : [num_layers][num_seqs][num_q_heads][window][head_dim]
 *                     query head j belongs to kv head j / (num_q_heads / num_kv_heads)
 *   scores, I, R    : float32 [num_layers][num_seqs][num_kv_heads][score_stride]
 *   keep            : int32   [num_layers][num_seqs][num_kv_heads][budget]
 */
#ifndef RKV_H_
#define RKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rkv_status {
  RKV_OK = 0,
  RKV_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent arguments   */
  RKV_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the kernels handle  */
  RKV_ERR_WORKSPACE = 3,    /* workspace missing or too small                   */
  RKV_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed       */
  RKV_ERR_DEVICE_CHECK = 5  /* a check on the device failed (rkv_device_status) */
} rkv_status;

typedef enum rkv_dtype { RKV_DTYPE_F32 = 0, RKV_DTYPE_BF16 = 1 } rkv_dtype;
typedef enum rkv_layout { RKV_LAYOUT_CONTIGUOUS = 0, RKV_LAYOUT_PAGED = 1 } rkv_layout;

/* Status word flags (rkv_device_status). */
#define RKV_DEVICE_SPAN_TIMEOUT 1u  /* a key-span wait reached its bound           */
#define RKV_DEVICE_BAD_BLOCK_ID 2u  /* a block-table id outside [0, num_blocks)    */

/* Longest cache (tokens per sequence) the kernels accept. */
#define RKV_MAX_LEN 32768
/* Largest num_q_heads / num_kv_heads * window the scoring kernels accept. */
#define RKV_MAX_WINDOW_ROWS 142

/* The method's knobs (the HF flags kv_budget, window_size, mix_lambda and
 * divide_length on the R-KV project page, section "Installing R-KV and running
 * a first math evaluation"; budget and buffer as in "How R-KV decides what to
 * drop") plus the model and cache shape. */
typedef struct rkv_config {
  int32_t num_layers;     /* >= 1                                               */
  int32_t num_q_heads;    /* >= 1, a multiple of num_kv_heads                   */
  int32_t num_kv_heads;   /* >= 1                                               */
  int32_t head_dim;       /* 64 or 128                                          */
  int32_t budget;         /* B > window: tokens kept per unit, window included  */
  int32_t buffer;         /* > 0: a sequence triggers iff len >= budget+buffer  */
  int32_t window;         /* w >= 1: window queries, and tokens always kept     */
  float mix_lambda;       /* lambda in [0, 1]                                   */
  int32_t dtype;          /* rkv_dtype of K, V and the window queries           */
  int32_t layout;         /* rkv_layout of K and V                              */
  int32_t block_size;     /* paged: tokens per block (>= 1); ignored otherwise  */
  int32_t shared_selection; /* 0: each KV head keeps its own budget tokens.
                               1: the KV heads of a (sequence, layer) keep one
                               common set, ranked by the sum of their scores
                               (head 0 + head 1 + ... in float32, in that order)
                               -- the identical eviction the R-KV project page
                               describes for tensor-parallel ranks ("How R-KV
                               decides what to drop").  Scores are still per
                               head; every head's keep row holds the same list. */
  int32_t check_block_table; /* paged, 0 or 1.  1: before any kernel reads the
                               pool, every block id a triggered sequence uses
                               (logical blocks [0, ceil(len / block_size))) is
                               checked against [0, num_blocks); a bad id sets
                               RKV_DEVICE_BAD_BLOCK_ID and no kernel of the
                               call reads or writes the pool.  Needs a
                               workspace in every call that reads the pool
                               (rkv_redundancy_gram does not check). */
} rkv_config;

/* The KV cache the step reads and compacts (device memory, caller-owned). */
typedef struct rkv_cache {
  void *k;                          /* keys   (layout above)                    */
  void *v;                          /* values (same layout as k)                */
  int64_t layer_stride;             /* elements from one layer to the next, for
                                       K and V alike; 0 = packed.  Otherwise at
                                       least the packed layer size (S*Hkv*cap*d
                                       or num_blocks*Hkv*block_size*d) and a
                                       multiple of 16 bytes, so that layers
                                       padded apart in one allocation are used
                                       in place (the R-KV project page, "How
                                       R-KV decides what to drop", scores all
                                       layers in one batched pass).             */
  int32_t capacity;                 /* contiguous: token slots per (l, s, h)    */
  int32_t num_blocks;               /* paged: blocks per layer in the pool      */
  const int32_t *block_table;       /* paged: device int32 [num_seqs][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;       /* paged                                    */
} rkv_cache;

/* Text of a status code (static storage). */
const char *rkv_status_string(rkv_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char *rkv_last_error(void);

/* 1 if a sequence of `len` cached tokens triggers (len >= budget + buffer),
 * else 0; the rule of "How R-KV decides what to drop".  Returns -1 if cfg is
 * NULL. */
int32_t rkv_is_triggered(const rkv_config *cfg, int32_t len);

/* Bytes of device workspace rkv_score needs for any batch of at most
 * num_seqs sequences of at most max_len tokens.  0 on invalid arguments.
 * The first 256 bytes hold the status word (rkv_device_status); the same
 * workspace is then passed to rkv_select and rkv_compact. */
size_t rkv_workspace_size(const rkv_config *cfg, int32_t num_seqs, int32_t max_len);

/* Step 1, scoring: I, R and S of every cached token of every triggered unit,
 * all layers in one pass ("batched cross-layer scoring" on the R-KV project
 * page; the two signals and their blend in the blog's R-KV section).
 *   q_window   device, window queries (layout above)
 *   h_seq_lens host int32 [num_seqs], current cache lengths
 *   scores     device float32 (layout above), columns [0, len) of triggered
 *              rows written; score_stride >= the longest triggered length
 *   importance, redundancy  device float32 like scores, or NULL to skip
 *   workspace  device, >= rkv_workspace_size(cfg, num_seqs, max len), 256-byte
 *              aligned; contents on entry are ignored.  The call clears its
 *              status word, then records what its kernels find there.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED (head_dim, window rows,
 * length above RKV_MAX_LEN), RKV_ERR_WORKSPACE, RKV_ERR_HIP. */
rkv_status rkv_score(const rkv_config *cfg, const rkv_cache *cache, const void *q_window,
                     int32_t num_seqs, const int32_t *h_seq_lens,
                     float *scores, int32_t score_stride,
                     float *importance, float *redundancy,
                     void *workspace, size_t workspace_bytes, void *stream);

/* The window-query ring of the decode loop: the last `window` queries of each
 * sequence, which the scoring calls read as q_window ("How R-KV decides what
 * to drop": the last window_size queries score the cache).  Decode step t of
 * sequence s stores its queries (every query head) into slot t mod window of
 * q_window, for layers layer0 .. layer0 + layer_count - 1; after any window
 * consecutive steps the ring holds exactly the last window queries.  The
 * scoring averages over the window rows, so their rotated order does not
 * change any result beyond float rounding.  The slot is computed on the GPU,
 * so the call can be captured in a decode graph.
 *   q_step    device, the step's queries [layer_count][num_seqs][num_q_heads][head_dim]
 *             in the cache dtype, 16-byte aligned
 *   d_steps   device int32 [num_seqs]: each sequence's decode step counter
 *             (any integer; a counter that keeps counting across compaction,
 *             unlike the cache length, which drops to `budget`)
 *   q_window  device, [num_layers][num_seqs][num_q_heads][window][head_dim]
 *             (the layout of rkv_score's q_window), 16-byte aligned; only the
 *             slot of each (layer, sequence, head) is written
 * Errors: RKV_ERR_INVALID_ARG (NULL, misaligned, layers outside
 * [0, num_layers)), RKV_ERR_UNSUPPORTED (as for the config), RKV_ERR_HIP. */
rkv_status rkv_window_store(const rkv_config *cfg, int32_t layer0, int32_t layer_count,
                            const void *q_step, int32_t num_seqs, const int32_t *d_steps,
                            void *q_window, void *stream);

/* The redundancy signal alone, through the explicit cosine Gram matrix: for
 * every key j of every triggered unit, R_j = the mean of cos(k_j, k_i) over
 * the unit's other keys i, with cos = 0 against a zero key -- the mean
 * off-diagonal entry of row j of the unit's N x N cosine matrix (R-KV project
 * page, "How R-KV decides what to drop"; the blog's R-KV section).  Every one
 * of the N^2 d products is formed on the matrix cores, from the cached bf16
 * keys themselves with float32 sums; the 1/|k| factors are applied in float32.
 * The values equal rkv_score's redundancy output up to rounding (that call
 * uses the equivalent rank-one form).  No workspace.
 *   cache       bf16 keys (v is not read)
 *   h_seq_lens  host int32 [num_seqs], current cache lengths (not modified)
 *   redundancy  device float32, laid out as rkv_score's scores, columns
 *               [0, len) of triggered rows written; stride >= the longest
 *               triggered length
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED (float32 caches, head_dim,
 * length above RKV_MAX_LEN), RKV_ERR_HIP. */
rkv_status rkv_redundancy_gram(const rkv_config *cfg, const rkv_cache *cache, int32_t num_seqs,
                               const int32_t *h_seq_lens, float *redundancy, int32_t stride,
                               void *stream);

/* Step 2, selection ("How R-KV decides what to drop" on the R-KV project
 * page: the last window_size tokens stay, the budget bounds what is kept; the
 * blog's R-KV section: tokens of high importance and low redundancy are the
 * ones kept): for each triggered unit, keep[0 .. budget-window) = the
 * chosen candidates of [0, len-window) in ascending position order, and
 * keep[budget-window .. budget) = len-window .. len-1 (the window).  Candidates
 * are ranked by score descending, ties by lower position; -0.0 ranks equal to
 * +0.0.  NaN scores give an unspecified (but in-range, duplicate-free) set.
 * With cfg->shared_selection = 1 the ranking score of a token is the float32
 * sum of its scores over the KV heads of its (sequence, layer), and all those
 * heads receive the same keep row.
 *   scores     device float32 (layout above), as written by rkv_score
 *   keep       device int32 (layout above)
 *   workspace  the workspace rkv_score used, or NULL: with a nonzero status
 *              word the keep rows are not written.  workspace_bytes >= 256.
 * Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE,
 * RKV_ERR_HIP. */
rkv_status rkv_select(const rkv_config *cfg, int32_t num_seqs, const int32_t *h_seq_lens,
                      const float *scores, int32_t score_stride, int32_t *keep,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Step 3, compaction and FREE_BLOCKS ("two-phase compaction" and
 * "bounded-footprint block freeing" on the R-KV project page): for each
 * triggered unit, K and V slot i receive the row of token keep[i], in place;
 * rows at slots >= budget are left as they were.  Then h_seq_lens[s] = budget
 * for each triggered s.
 * Paged layout: the physical ids of logical blocks ceil(budget/block_size) ..
 * ceil(len/block_size)-1 of each triggered sequence are written to
 * free_blocks (device int32), sequences in order, blocks in logical order;
 * h_free_counts[s] (host, may be NULL) receives the count per sequence (0 for
 * sequences not triggered).  The block table is not modified: returning the
 * ids to an allocator is the caller's.  free_capacity = entries available in
 * free_blocks.  Contiguous layout: free_blocks may be NULL; counts are 0.
 *   keep       device int32 (layout above), ascending per unit, as from rkv_select
 *   workspace  the workspace rkv_score used, or NULL.  Given, a nonzero
 *              status word leaves the cache and free_blocks untouched (the
 *              host lengths and counts are still updated: after a nonzero
 *              rkv_device_status the caller restores the lengths it passed).
 *              With cfg->check_block_table = 1 it is required, and the block
 *              ids are checked again before the pool is touched.
 *              workspace_bytes >= 256.
 * Errors: RKV_ERR_INVALID_ARG (including free_capacity too small),
 * RKV_ERR_UNSUPPORTED, RKV_ERR_WORKSPACE, RKV_ERR_HIP.  A keep row that is
 * not strictly ascending within [0, len) is undefined behaviour. */
rkv_status rkv_compact(const rkv_config *cfg, const rkv_cache *cache, int32_t num_seqs,
                       int32_t *h_seq_lens, const int32_t *keep,
                       int32_t *free_blocks, int32_t free_capacity,
                       int32_t *h_free_counts, void *workspace, size_t workspace_bytes,
                       void *stream);

/* The whole step in one call: the outputs of rkv_score (scores only),
 * rkv_select and rkv_compact, with the same arguments and the same results
 * bit for bit.  For bf16 units of up to 1280 keys (head_dim 128; 2560 at 64)
 * with num_q_heads / num_kv_heads * window <= 78 and per-head selection
 * (shared_selection = 0), one kernel per launch
 * scores, selects and compacts each unit, keeping its keys on chip so the
 * keys are read from HBM once; other launches run the three kernels in
 * order (R-KV project page, "How R-KV differs from static KV cache
 * compression": the scoring work sits on the decode critical path, which is
 * why it is fused where it fits).
 *   h_seq_lens  host, in/out (triggered sequences become `budget` long)
 *   workspace   as for rkv_score; launches that cannot run fused use it for
 *               their scoring records.  NULL is accepted when every launch
 *               runs fused and cfg->check_block_table = 0; given, its status
 *               word is cleared and then set as for the three calls.
 * Errors: the union of those of the three calls. */
rkv_status rkv_step(const rkv_config *cfg, const rkv_cache *cache, const void *q_window,
                    int32_t num_seqs, int32_t *h_seq_lens,
                    float *scores, int32_t score_stride, int32_t *keep,
                    int32_t *free_blocks, int32_t free_capacity, int32_t *h_free_counts,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace rkv_step_device needs for num_seqs sequences of
 * lengths up to max_len (the triggered-sequence table, plus the scoring
 * records when the launch cannot run fused).  0 on invalid arguments. */
size_t rkv_step_device_workspace_size(const rkv_config *cfg, int32_t num_seqs, int32_t max_len);

/* rkv_step with the sequence lengths in device memory, for a step that runs
 * inside a captured decode graph (the in-graph decode the R-KV project page
 * names for its vLLM port, section "How R-KV differs from static KV cache
 * compression"): the host
 * takes no decision that depends on the lengths, every launch has a shape
 * fixed by (num_seqs, max_len), and the trigger is taken on the GPU.
 * Results are those of rkv_step for the same lengths, bit for bit.
 *   d_seq_lens    device int32 [num_seqs], in/out: triggered sequences
 *                 (budget + buffer <= len <= max_len) become `budget` long.
 *                 A length above max_len is left alone (not compressed).
 *   max_len       host: upper bound of the lengths this call may compress;
 *                 sizes the launches and the workspace.  <= RKV_MAX_LEN, and
 *                 <= capacity (contiguous) or max_blocks_per_seq * block_size
 *                 (paged).  score_stride >= max_len.
 *   free_blocks   paged: as for rkv_compact; free_capacity must cover every
 *                 sequence triggering at max_len:
 *                 num_seqs * (ceil(max_len/bs) - ceil(budget/bs)) entries.
 *   d_free_counts device int32 [num_seqs] or NULL: freed blocks per sequence.
 *   workspace     device, >= rkv_step_device_workspace_size(cfg, num_seqs,
 *                 max_len) bytes, 256-byte aligned; contents on entry ignored.
 *                 Its status word is set as for rkv_step; a nonzero word
 *                 leaves the cache, the keep rows and free_blocks untouched
 *                 (the device lengths and counts are still updated).
 * Errors: those of rkv_step, checked on the host before anything is enqueued
 * (lengths are not read by the host). */
rkv_status rkv_step_device(const rkv_config *cfg, const rkv_cache *cache, const void *q_window,
                           int32_t num_seqs, int32_t *d_seq_lens, int32_t max_len,
                           float *scores, int32_t score_stride, int32_t *keep,
                           int32_t *free_blocks, int32_t free_capacity, int32_t *d_free_counts,
                           void *workspace, size_t workspace_bytes, void *stream);

/* The KARA-style sliding-window variant (the KARA entry on the fugumt.com
 * paper page, "KARA: Efficient Reasoning LLM Serving via Sliding-Window KV
 * Cache Compression", Abstract: decode-time compression of only the recently
 * generated context, bidirectional attention to score the window's KV pairs,
 * Token2Chunk widening some of the selected pairs into chunks).  The
 * abstract gives no formulas; this library reads it as follows. */
typedef struct rkv_kara_config {
  int32_t window_len;  /* W: the tail compressed at once (32, 64 or 128 tokens)   */
  int32_t keep;        /* K in [1, W]: window tokens kept                         */
  int32_t anchors;     /* m >= 0: the best tokens widened into chunks             */
  int32_t radius;      /* r >= 0: a chunk is the positions within r of an anchor;
                          m * (2 r + 1) <= K                                      */
} rkv_kara_config;

/* One KARA-style step.  A sequence triggers once its uncompressed tail
 * (tokens from h_tail_start[s] on) holds W tokens; its window is then the
 * last W tokens, t0 = len - W .. len - 1.  Per (sequence, layer, kv head):
 *   score_j = mean over the G*W query rows (the window tokens' queries of the
 *             G query heads that share the kv head) of softmax_j(q . k_j /
 *             sqrt(d)) over the W window keys -- bidirectional: no causal mask;
 *   keep    = the chunks [a - r, a + r] (clipped to the window) of the m best
 *             tokens a, then the best tokens outside those chunks until K
 *             places are filled (equal scores: lower position first);
 *   slots t0 .. t0 + K - 1 of K and V receive the kept tokens' rows in
 *   position order; the prefix [0, t0) is not touched.
 * Then h_seq_lens[s] = h_tail_start[s] = t0 + K.  Every kv head keeps its own
 * set.  cfg gives the model and cache shape (bf16 caches; budget, buffer,
 * window, mix_lambda and shared_selection are not used).
 *   q_tail        device bf16 [num_layers][num_seqs][num_q_heads][W][head_dim]:
 *                 the queries of the window tokens, any order within a head
 *                 (rkv_window_store with window = W keeps them)
 *   h_seq_lens, h_tail_start  host int32 [num_seqs], in/out
 *   scores        device float32 [num_layers][num_seqs][num_kv_heads][W]
 *   keep          device int32 [num_layers][num_seqs][num_kv_heads][K]: the
 *                 kept tokens' positions (t0 + window index), ascending
 *   free_blocks   paged: ids of logical blocks ceil((t0+K)/bs) ..
 *                 ceil(len/bs) - 1, sequences in order; h_free_counts as for
 *                 rkv_compact
 *   workspace     NULL, or >= 256 bytes (256-byte aligned) whose status word
 *                 records a failed block-id check; required with
 *                 cfg->check_block_table = 1
 * Rows, scores and keep entries of sequences that do not trigger are not
 * written.  Errors: RKV_ERR_INVALID_ARG, RKV_ERR_UNSUPPORTED (float32, W,
 * head_dim, length above RKV_MAX_LEN), RKV_ERR_WORKSPACE, RKV_ERR_HIP. */
rkv_status rkv_kara_step(const rkv_config *cfg, const rkv_kara_config *kc, const rkv_cache *cache,
                         const void *q_tail, int32_t num_seqs, int32_t *h_seq_lens,
                         int32_t *h_tail_start, float *scores, int32_t *keep,
                         int32_t *free_blocks, int32_t free_capacity, int32_t *h_free_counts,
                         void *workspace, size_t workspace_bytes, void *stream);

/* rkv_step without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments as rkv_step minus the workspace, same
 * results bit for bit.  The scratch the step needs (the status word and the
 * scoring records of launches that cannot run fused) lives in a 32 MiB
 * device array of the library, one per GPU, held from the first call on that
 * GPU until the process ends; the call allocates nothing.  Calls that
 * overlap on one GPU (other streams, other host threads) share that array
 * and race: keep them on one stream.  Its status word is read with
 * rkv_device_status(NULL, ...).
 * Errors: those of rkv_step; RKV_ERR_WORKSPACE when a launch that cannot run
 * fused needs more than the 32 MiB (rkv_workspace_size for at most 128
 * triggered sequences of the longest length, e.g. 8 sequences of 4352 keys
 * of the paged Llama-8B workload take 25.5 MiB). */
rkv_status rkv_step_noalloc(const rkv_config *cfg, const rkv_cache *cache, const void *q_window,
                            int32_t num_seqs, int32_t *h_seq_lens,
                            float *scores, int32_t score_stride, int32_t *keep,
                            int32_t *free_blocks, int32_t free_capacity, int32_t *h_free_counts,
                            void *stream);

/* The status word of a workspace (its first 32-bit word) after the calls
 * enqueued on `stream` so far: waits for the stream, then copies the word to
 * the host (so it cannot be captured in a graph).  *flags (may be NULL)
 * receives it: RKV_DEVICE_SPAN_TIMEOUT, RKV_DEVICE_BAD_BLOCK_ID or 0.
 * Returns RKV_OK for 0, RKV_ERR_DEVICE_CHECK otherwise (the step left the
 * cache as it was; see rkv_compact for the lengths).  workspace NULL: the
 * word of rkv_step_noalloc's scratch on the current device.
 * Errors: RKV_ERR_HIP. */
rkv_status rkv_device_status(const void *workspace, void *stream, uint32_t *flags);

/* Bound of the key-span wait, in microseconds, for launches enqueued after
 * this call by any thread (default 1000000, at most 60000000).  0 makes every
 * key span give up at once and report RKV_DEVICE_SPAN_TIMEOUT, which
 * exercises the failure path.  Returns the previous bound, or -1 (nothing
 * changed) for an argument outside [0, 60000000]. */
int64_t rkv_set_span_wait_us(int64_t microseconds);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H_ */
