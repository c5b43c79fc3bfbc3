"""CPU oracle for the R-KV decode-time KV-cache compression step.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never calls it, and this module imports
nothing from the product path.

Plain, slow, float64.  Every function follows one step of the method as the
pages describe it; where they are silent the plainest reading is taken and
named in the docstring.  Sources:

* [PROJ] R-KV project page (hysenlabs.com, "R-KV: Redundancy-Aware KV Cache
  Compression for Reasoning Models"): section "How R-KV decides what to drop:
  budget, buffer and cross-layer scoring" (decode-time trigger on budget and
  buffer, a local window, mix_lambda blending two scores, FREE_BLOCKS
  returning evicted blocks), and the command block of "Installing R-KV and
  running a first math evaluation" (kv_budget 1024, window_size 8,
  mix_lambda 0.1, divide_length 128).
* [BLOG] hotdry blog post on R-KV, EvolKV and Ada-KV, section on R-KV:
  redundancy from cosine similarity of key vectors, importance from
  multi-head attention, eviction that favours high importance and low
  redundancy, lambda near 0.1.  Section on risks: pure attention scoring
  (SnapKV-like) is the lambda = 1 case.

Numbers: bf16 inputs are widened exactly to float64; all arithmetic is float64.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

__all__ = [
    "decode", "is_triggered", "window_logits", "importance", "cosine_gram",
    "redundancy", "mixed_score", "score_unit", "select_keep", "compact_rows",
    "free_blocks", "unit_step", "q_group", "step_unit",
    "shared_score", "select_keep_shared", "layer_step_shared", "redundancy_at",
    "window_store",
]


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float64.  bf16 is stored as its 16 bit pattern, which
    is the top half of the float32 with the same value."""
    if dtype == "bf16":
        w = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return w.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def is_triggered(n: int, budget: int, buffer: int) -> bool:
    """[PROJ] "How R-KV decides what to drop": compression runs at decode time
    once the cache has grown by a buffer beyond the budget.  Reading: a
    sequence of n cached tokens triggers iff n >= budget + buffer (with the
    HF path's step_length division, buffer = divide_length)."""
    return int(n) >= int(budget) + int(buffer)


def window_logits(q_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Scaled dot products q.k / sqrt(d) of the window queries against every
    cached key: (G*w, d) x (N, d) -> (G*w, N)."""
    d = k.shape[1]
    return (q_rows @ k.T) / math.sqrt(d)


def importance(q_rows: np.ndarray, k: np.ndarray) -> np.ndarray:
    """[BLOG] R-KV section: importance of a cached token comes from the
    attention the model pays it; [PROJ]: the last window_size queries do the
    scoring.  Reading: each of the G*w rows (the window's queries of every
    query head sharing this kv head) is a softmax over all N cached keys, no
    causal mask inside the window, scale 1/sqrt(d); the importance of token j
    is the mean of its attention weight over those rows."""
    logits = window_logits(q_rows, k)
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


def cosine_gram(k: np.ndarray) -> np.ndarray:
    """[BLOG] R-KV section: redundancy is measured by cosine similarity between
    key vectors.  Returns the N x N matrix of cosines of the L2-normalised keys
    (a zero key normalises to the zero vector)."""
    norms = np.sqrt((k * k).sum(axis=1))
    safe = np.where(norms > 0, norms, 1.0)
    khat = np.where(norms[:, None] > 0, k / safe[:, None], 0.0)
    return khat @ khat.T


def redundancy(k: np.ndarray) -> np.ndarray:
    """Mean off-diagonal cosine similarity of each key to the other N - 1 keys
    of the same (sequence, layer, kv head), over all N keys (window included)."""
    n = k.shape[0]
    assert n >= 2
    c = cosine_gram(k)
    off = c.sum(axis=1) - np.diag(c)
    return off / (n - 1)


def redundancy_at(k: np.ndarray, idx) -> np.ndarray:
    """The redundancy of the tokens idx only, for caches too long for the
    N x N Gram: for each j, row j of the cosine matrix (the cosines of key j
    with every key), minus its diagonal entry, over N - 1.  The same
    definition as redundancy(), one row at a time."""
    n = k.shape[0]
    assert n >= 2
    norms = np.sqrt((k * k).sum(axis=1))
    safe = np.where(norms > 0, norms, 1.0)
    khat = np.where(norms[:, None] > 0, k / safe[:, None], 0.0)
    out = []
    for j in np.asarray(idx, dtype=np.int64):
        row = khat @ khat[j]
        out.append((row.sum() - row[j]) / (n - 1))
    return np.array(out, dtype=np.float64)


def mixed_score(imp: np.ndarray, red: np.ndarray, lam: float) -> np.ndarray:
    """[PROJ] mix_lambda blends the two signals; [BLOG] keep high importance
    and low redundancy.  S = lam * I - (1 - lam) * R, larger is kept.  No
    normalisation of either score before mixing (none is described)."""
    return lam * imp - (1.0 - lam) * red


def score_unit(q_rows: np.ndarray, k: np.ndarray, lam: float):
    """(I, R, S) for one (sequence, layer, kv head)."""
    imp = importance(q_rows, k)
    red = redundancy(k)
    return imp, red, mixed_score(imp, red, lam)


def select_keep(scores: np.ndarray, n: int, budget: int, window: int) -> np.ndarray:
    """Keep set of one unit: the last `window` tokens always, plus the
    budget - window best candidates of [0, n - window) ranked by score
    descending, equal scores broken by lower position first.  Returned in
    ascending position order (slot i of the compacted cache holds keep[i]).
    Reading: the budget counts the window ([PROJ] names budget and window
    separately; the compacted cache then holds exactly `budget` tokens)."""
    assert 0 < window < budget <= n
    cand = n - window
    s = np.asarray(scores[:cand], dtype=np.float64)
    pos = np.arange(cand)
    order = np.lexsort((pos, -s))          # primary: -s ascending; then position
    chosen = np.sort(order[: budget - window])
    return np.concatenate([chosen, np.arange(cand, n)]).astype(np.int64)


def shared_score(head_scores: np.ndarray) -> np.ndarray:
    """Head-shared mode.  [PROJ] "How R-KV decides what to drop": under tensor
    parallelism every rank evicts the identical token set.  Reading: the KV
    heads of one (sequence, layer) rank the tokens by the sum of their mixed
    scores S_h (an (H, N) array -> N); the sum, not a mean, so the ranking
    needs no division (a mean ranks identically)."""
    hs = np.asarray(head_scores, dtype=np.float64)
    return hs.sum(axis=0)


def select_keep_shared(head_scores: np.ndarray, n: int, budget: int, window: int) -> np.ndarray:
    """One keep set for all KV heads of a (sequence, layer): the per-unit
    rule of select_keep applied to the summed scores."""
    return select_keep(shared_score(head_scores), n, budget, window)


def compact_rows(rows: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Slot i of the compacted cache receives row keep[i] ([PROJ]: two-phase
    compaction of the kept entries).  Plain fancy indexing."""
    return rows[np.asarray(keep)]


def free_blocks(bt_row: Sequence[int], n: int, budget: int, block_size: int) -> List[int]:
    """[PROJ] FREE_BLOCKS: blocks emptied by compaction go back to the
    allocator.  After compaction the sequence holds `budget` tokens in its
    first ceil(budget/bs) logical blocks; logical blocks ceil(budget/bs) ..
    ceil(n/bs)-1 are freed, reported as physical ids in logical order."""
    first = -(-budget // block_size)
    last = -(-n // block_size)
    return [int(bt_row[b]) for b in range(first, last)]


def unit_step(q_rows, k, k_store, v_store, budget, window, lam):
    """Everything one unit produces: I, R, S, keep, K', V'.  q_rows and k are
    float64; k_store and v_store are the same rows in storage dtype, so that
    the compacted rows are the input bits."""
    n = k.shape[0]
    imp, red, s = score_unit(q_rows, k, lam)
    keep = select_keep(s, n, budget, window)
    return dict(imp=imp, red=red, score=s, keep=keep,
                k_new=compact_rows(k_store, keep), v_new=compact_rows(v_store, keep))


def layer_step_shared(q_rows_per_head, k_per_head, k_store, v_store, budget, window, lam):
    """Head-shared mode for one (sequence, layer): I, R, S of every KV head
    as in unit_step, one keep set from the summed S, and every head's K and
    V compacted with it.  Arguments are per-head lists (float64 q rows and
    keys; storage-dtype key and value rows)."""
    heads = [score_unit(q, k, lam) for q, k in zip(q_rows_per_head, k_per_head)]
    n = k_per_head[0].shape[0]
    keep = select_keep_shared(np.stack([h[2] for h in heads]), n, budget, window)
    return [dict(imp=imp, red=red, score=sc, keep=keep,
                 k_new=compact_rows(ks, keep), v_new=compact_rows(vs, keep))
            for (imp, red, sc), ks, vs in zip(heads, k_store, v_store)]


def window_store(q_window: np.ndarray, q_step: np.ndarray, layer0: int, steps, window: int) -> np.ndarray:
    """[PROJ] "How R-KV decides what to drop": the last window_size queries of
    a sequence score its cache.  Reading: they are kept in a ring of `window`
    slots per (layer, sequence, query head); decode step t of sequence s
    writes its query into slot t mod window, so after any window consecutive
    steps the ring holds exactly the last window queries (in rotated order,
    which importance() does not see: it averages over the rows).
    q_window (L, S, Hq, w, d), q_step (count, S, Hq, d) for layers
    layer0 .. layer0 + count - 1; returns the updated copy (a bit copy)."""
    out = np.array(q_window, copy=True)
    for i in range(q_step.shape[0]):
        for s in range(q_step.shape[1]):
            out[layer0 + i, s, :, int(steps[s]) % window, :] = q_step[i, s]
    return out


def q_group(q_seq_layer: np.ndarray, h: int, group: int) -> np.ndarray:
    """Window-query rows of the query heads that share kv head h (GQA: query
    head j uses kv head j // group): (group, w, d) -> (group*w, d)."""
    qg = q_seq_layer[h * group:(h + 1) * group]
    return qg.reshape(-1, qg.shape[-1])


def step_unit(spec, q_sl, k_rows, v_rows, h):
    """One unit given its window queries (Hq, w, d) and its N key and value
    rows in logical order (storage dtype), e.g. gathered from a paged pool."""
    group = spec.num_q_heads // spec.num_kv_heads
    qd = decode(q_sl, spec.dtype)
    return unit_step(q_group(qd, h, group), decode(k_rows, spec.dtype), k_rows, v_rows,
                     spec.budget, spec.window, spec.mix_lambda)
