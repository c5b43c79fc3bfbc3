"""CPU oracle of the KARA-style sliding-window compression step.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the product path never calls
it, and it imports nothing from the product path.

Source: the KARA entry on the fugumt.com paper page ("KARA: Efficient
Reasoning LLM Serving via Sliding-Window KV Cache Compression"), Abstract.
The abstract names the parts and gives no formula; each function below takes
the plainest reading the rest of the abstract supports:

* decoding-time compression that operates only on the recently generated
  context: the window is the last `window_len` tokens of a sequence, taken
  once that many tokens have been generated since the previous compression
  (the R-KV knob divide_length plays that role in the workloads); the tokens
  before the window, compressed earlier, are not touched again;
* bidirectional attention scores and selects the KV pairs in the window:
  every window token's query attends to every window key with no causal
  mask (softmax over the window's keys, scale 1/sqrt(d)); a token's score is
  the mean of its attention weight over the rows of all query heads that
  share its KV head (grouped-query attention), as R-KV averages its window;
* Token2Chunk expands a subset of the selected pairs into chunks: the
  `anchors` best-scoring tokens are each widened to the chunk of positions
  within `radius` of it (clipped to the window); the remaining places of the
  window's `keep` are taken by the best other tokens; ties rank the lower
  position first;
* compaction keeps the prefix and packs the window's kept tokens right after
  it, in position order; paged caches free the blocks past the new length.

Plain float64; bf16 inputs are widened exactly.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

__all__ = ["is_triggered", "window_scores", "rank_order", "token2chunk_keep", "new_length",
           "free_blocks", "unit_step", "step_unit", "q_group_window"]


def is_triggered(n: int, tail_start: int, window_len: int) -> bool:
    """A sequence of n tokens whose uncompressed tail starts at tail_start is
    compressed once the tail holds window_len tokens."""
    return int(n) - int(tail_start) >= int(window_len)


def window_scores(q_rows: np.ndarray, k_window: np.ndarray) -> np.ndarray:
    """Bidirectional attention inside the window: (R, d) query rows against
    the (W, d) window keys; each row a softmax over all W keys (no mask),
    scale 1/sqrt(d); the score of key j is its weight averaged over the R
    rows."""
    d = k_window.shape[1]
    logits = (q_rows @ k_window.T) / math.sqrt(d)
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


def rank_order(scores: np.ndarray) -> np.ndarray:
    """Window positions from best to worst: score descending, then position
    ascending."""
    s = np.asarray(scores, dtype=np.float64)
    return np.lexsort((np.arange(len(s)), -s))


def token2chunk_keep(scores: np.ndarray, keep: int, anchors: int, radius: int) -> np.ndarray:
    """The kept window positions (ascending, exactly `keep` of them): the
    chunks [a - radius, a + radius] (clipped to the window) around the
    `anchors` best tokens a, then the best tokens outside every chunk until
    `keep` places are filled.  Requires anchors * (2 radius + 1) <= keep."""
    w = len(scores)
    assert 0 < keep <= w and anchors * (2 * radius + 1) <= keep
    order = rank_order(scores)
    in_chunk = np.zeros(w, dtype=bool)
    for a in order[:anchors]:
        in_chunk[max(0, a - radius): min(w, a + radius + 1)] = True
    rest = [int(j) for j in order if not in_chunk[j]]
    kept = in_chunk.copy()
    kept[rest[: keep - int(in_chunk.sum())]] = True
    return np.flatnonzero(kept).astype(np.int64)


def new_length(n: int, window_len: int, keep: int) -> int:
    """Length after compressing the last window_len of n tokens to keep."""
    return int(n) - int(window_len) + int(keep)


def free_blocks(bt_row: Sequence[int], n: int, n_new: int, block_size: int) -> List[int]:
    """Paged layout: logical blocks ceil(n_new / bs) .. ceil(n / bs) - 1 hold no
    token after compaction; their physical ids, in logical order."""
    first = -(-int(n_new) // block_size)
    last = -(-int(n) // block_size)
    return [int(bt_row[b]) for b in range(first, last)]


def unit_step(q_rows, k_window, k_store, v_store, keep, anchors, radius):
    """One (sequence, layer, kv head): scores of the window, the kept window
    positions, and the window's new rows (storage dtype) for slots 0 .. keep-1
    after the prefix."""
    s = window_scores(q_rows, k_window)
    kept = token2chunk_keep(s, keep, anchors, radius)
    return dict(score=s, keep=kept, k_new=k_store[kept], v_new=v_store[kept])


def q_group_window(q_seq_layer: np.ndarray, h: int, group: int) -> np.ndarray:
    """The window queries of the query heads sharing kv head h (GQA: query
    head j uses kv head j // group): (Hq, W, d) -> (group * W, d)."""
    qg = q_seq_layer[h * group:(h + 1) * group]
    return qg.reshape(-1, qg.shape[-1])


def _decode(x, dtype):
    if dtype == "bf16":
        w = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return w.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def step_unit(kc, dtype, num_q_heads, num_kv_heads, q_tail_sl, k_rows, v_rows, h):
    """One unit from storage-dtype inputs: q_tail_sl (Hq, W, d) the queries of
    the window tokens, k_rows / v_rows (n, d) the unit's rows in logical
    order; kc has window_len, keep, anchors, radius.  keep positions are
    window-relative."""
    group = num_q_heads // num_kv_heads
    n = k_rows.shape[0]
    w = kc.window_len
    kw, vw = k_rows[n - w:n], v_rows[n - w:n]
    q = q_group_window(_decode(q_tail_sl, dtype), h, group)
    return unit_step(q, _decode(kw, dtype), kw, vw, kc.keep, kc.anchors, kc.radius)
