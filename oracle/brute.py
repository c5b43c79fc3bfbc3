"""Scalar brute force for tiny inputs — TEST INFRASTRUCTURE ONLY.

Pure-Python loops over lists of floats, written separately from the numpy
oracle in this package so that the two can check each other (only tests may
import it).  Follows the same readings of the R-KV pages (R-KV project page on
hysenlabs.com, section "How R-KV decides what to drop"; hotdry blog post,
R-KV section):

* importance: softmax over all cached keys of each window-query row,
  scale 1/sqrt(d), mean over rows;
* redundancy: mean cosine similarity to the other keys;
* mixed score lam*I - (1-lam)*R;
* selection by counting, for each candidate, how many candidates beat it
  (higher score, or equal score at a lower position) -- no sorting;
* compaction by copying row keep[i] to slot i.

Only for inputs with a few hundred keys at most.
"""
from __future__ import annotations

import math
from typing import List, Sequence

Row = Sequence[float]


def _dot(a: Row, b: Row) -> float:
    t = 0.0
    for x, y in zip(a, b):
        t += x * y
    return t


def importance(q_rows: Sequence[Row], keys: Sequence[Row]) -> List[float]:
    n = len(keys)
    d = len(keys[0])
    scale = 1.0 / math.sqrt(d)
    acc = [0.0] * n
    for q in q_rows:
        logits = [_dot(q, k) * scale for k in keys]
        top = max(logits)
        ex = [math.exp(x - top) for x in logits]
        z = 0.0
        for e in ex:
            z += e
        for j in range(n):
            acc[j] += ex[j] / z
    return [a / len(q_rows) for a in acc]


def redundancy(keys: Sequence[Row]) -> List[float]:
    n = len(keys)
    norms = [math.sqrt(_dot(k, k)) for k in keys]
    out = []
    for j in range(n):
        t = 0.0
        for i in range(n):
            if i == j or norms[i] == 0.0 or norms[j] == 0.0:
                continue
            t += _dot(keys[j], keys[i]) / (norms[j] * norms[i])
        out.append(t / (n - 1))
    return out


def mixed(imp: Sequence[float], red: Sequence[float], lam: float) -> List[float]:
    return [lam * a - (1.0 - lam) * b for a, b in zip(imp, red)]


def select_keep(scores: Sequence[float], n: int, budget: int, window: int) -> List[int]:
    cand = n - window
    want = budget - window
    keep = []
    for j in range(cand):
        beaten_by = 0
        for i in range(cand):
            if scores[i] > scores[j] or (scores[i] == scores[j] and i < j):
                beaten_by += 1
        if beaten_by < want:
            keep.append(j)
    keep.extend(range(cand, n))
    return keep


def select_keep_shared(head_scores: Sequence[Sequence[float]], n: int, budget: int,
                       window: int) -> List[int]:
    """Head-shared mode: sum the heads' scores token by token, then select."""
    total = []
    for j in range(n):
        t = 0.0
        for h in range(len(head_scores)):
            t += head_scores[h][j]
        total.append(t)
    return select_keep(total, n, budget, window)


def compact(rows: Sequence[Row], keep: Sequence[int]) -> List[Row]:
    out = []
    for i in range(len(keep)):
        out.append(list(rows[keep[i]]))
    return out


def free_blocks(bt_row: Sequence[int], n: int, budget: int, block_size: int) -> List[int]:
    """A logical block is freed when it held tokens before (its first token
    position < n) and holds none after compaction (first position >= budget)."""
    out = []
    b = 0
    while b * block_size < n:
        if b * block_size >= budget:
            out.append(int(bt_row[b]))
        b += 1
    return out


def unit(q_rows, keys, lam, budget, window):
    imp = importance(q_rows, keys)
    red = redundancy(keys)
    s = mixed(imp, red, lam)
    return imp, red, s, select_keep(s, len(keys), budget, window)


# ------------------------------------------------------------- KARA-style window step

def kara_scores(q_rows: Sequence[Row], keys: Sequence[Row]) -> List[float]:
    """Every row's softmax over all window keys (no mask), averaged over rows:
    the same loops as importance(), over the window's keys only."""
    return importance(q_rows, keys)


def kara_keep(scores: Sequence[float], keep: int, anchors: int, radius: int) -> List[int]:
    """Token2Chunk by counting: rank_j = how many positions beat j (higher
    score, or equal score at a lower position); anchors are the ranks below
    `anchors`; a position is in a chunk if an anchor lies within radius; the
    rest are taken in rank order among the positions outside every chunk."""
    w = len(scores)

    def beats(i, j):
        return scores[i] > scores[j] or (scores[i] == scores[j] and i < j)

    rank = [sum(1 for i in range(w) if beats(i, j)) for j in range(w)]
    in_chunk = [any(rank[a] < anchors and abs(a - j) <= radius for a in range(w)) for j in range(w)]
    left = keep - sum(in_chunk)
    out = []
    for j in range(w):
        if in_chunk[j]:
            out.append(j)
            continue
        better = sum(1 for i in range(w) if not in_chunk[i] and beats(i, j))
        if better < left:
            out.append(j)
    return out
