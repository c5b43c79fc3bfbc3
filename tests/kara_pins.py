"""Pins of the KARA-style window oracle (oracle/kara_oracle.py) against facts
that do not come from it: hand-worked examples (tests/golden/kara_examples.json),
invariants and closed forms of the readings, special cases that reduce to a
plain ranking, and the scalar brute force of oracle/brute.py.  Each pin takes
the oracle module, so the mutation test runs them against broken copies."""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "kara_examples.json")) as f:
        return json.load(f)


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.abs(a - b) <= tol * np.maximum(1.0, np.abs(b))), (a, b)


def _rand(seed, rows, w, d):
    rng = np.random.default_rng([78, seed])
    return rng.standard_normal((rows, d)), rng.standard_normal((w, d)) + rng.standard_normal(d) * 0.5


def pin_golden_scores(k):
    for ex in golden()["scores"]:
        _close(k.window_scores(np.array(ex["q"], float), np.array(ex["k"], float)), ex["expect"])


def pin_golden_select(k):
    for ex in golden()["select"]:
        got = k.token2chunk_keep(np.array(ex["scores"]), ex["keep"], ex["anchors"], ex["radius"])
        assert list(got) == ex["expect"], (ex["name"], got)


def pin_golden_lengths_and_trigger(k):
    g = golden()
    for ex in g["length"]:
        assert k.new_length(ex["n"], ex["window_len"], ex["keep"]) == ex["expect"]
    for ex in g["trigger"]:
        assert bool(k.is_triggered(ex["n"], ex["tail_start"], ex["window_len"])) == ex["expect"], ex
    for ex in g["free_blocks"]:
        row = list(range(1000, 1000 + ex["bt_row_len"]))
        got = k.free_blocks(row, ex["n"], ex["n_new"], ex["block_size"])
        assert got == [1000 + b for b in ex["expect_logical"]], (ex["name"], got)


def pin_scores_sum_to_one(k):
    """Each row is a softmax over the window, so the row mean sums to 1."""
    for seed, (rows, w, d) in enumerate([(8, 16, 8), (512, 128, 64), (6, 3, 4)]):
        q, kw = _rand(seed, rows, w, d)
        s = k.window_scores(q, kw)
        assert abs(s.sum() - 1.0) < 1e-12 and np.all(s > 0)


def pin_scale_one_over_sqrt_d(k):
    """Two orthonormal keys and one row a*e0: the weight of key 0 is
    1/(1 + exp(-a/sqrt(d))) whatever the padding dimension d."""
    for d in (2, 16, 128):
        kw = np.zeros((2, d))
        kw[0, 0] = kw[1, 1] = 1.0
        q = np.zeros((1, d))
        q[0, 0] = 3.0
        _close(k.window_scores(q, kw)[0], 1.0 / (1.0 + math.exp(-3.0 / math.sqrt(d))))


def pin_rows_are_exchangeable_and_keys_equivariant(k):
    """Bidirectional, unmasked attention: reordering the query rows changes
    nothing, and reordering the window's keys reorders the scores alike (a
    causal mask would tie the weights to the positions)."""
    q, kw = _rand(9, 12, 10, 8)
    s = k.window_scores(q, kw)
    rng = np.random.default_rng(3)
    _close(k.window_scores(q[rng.permutation(12)], kw), s, tol=1e-13)
    perm = rng.permutation(10)
    _close(k.window_scores(q, kw[perm]), s[perm], tol=1e-13)


def pin_brute_force_scores(k):
    for seed, (rows, w, d) in enumerate([(4, 6, 3), (16, 16, 8), (2, 33, 5)]):
        q, kw = _rand(20 + seed, rows, w, d)
        _close(k.window_scores(q, kw), brute.kara_scores(q.tolist(), kw.tolist()))


def pin_brute_force_select(k):
    """Random score rows, exact ties included, against the counting form."""
    rng = np.random.default_rng([78, 40])
    for trial in range(150):
        w = int(rng.integers(2, 40))
        r = int(rng.integers(0, 4))
        keep = int(rng.integers(1, w + 1))
        anchors = int(rng.integers(0, keep // (2 * r + 1) + 1))
        s = rng.integers(0, 6, size=w).astype(float) if trial % 3 == 0 else rng.standard_normal(w)
        got = list(k.token2chunk_keep(s, keep, anchors, r))
        assert got == brute.kara_keep(list(s), keep, anchors, r), (trial, s, keep, anchors, r)


def pin_select_invariants(k):
    """keep places exactly, ascending, inside the window; every anchor's chunk
    is kept; no anchors (or radius 0) is the plain best-keep ranking."""
    rng = np.random.default_rng([78, 41])
    for trial in range(100):
        w = int(rng.integers(4, 64))
        r = int(rng.integers(0, 3))
        keep = int(rng.integers(2 * r + 1, w + 1))
        anchors = int(rng.integers(1, keep // (2 * r + 1) + 1))
        s = rng.standard_normal(w)
        kept = k.token2chunk_keep(s, keep, anchors, r)
        assert len(kept) == keep and np.all(np.diff(kept) > 0) and kept[0] >= 0 and kept[-1] < w
        best = np.argsort(-s, kind="stable")
        for a in best[:anchors]:
            for j in range(max(0, a - r), min(w, a + r + 1)):
                assert j in kept
        plain = np.sort(best[:keep])
        assert list(k.token2chunk_keep(s, keep, 0, r)) == list(plain)
        assert list(k.token2chunk_keep(s, keep, min(anchors, keep), 0)) == list(plain)


def pin_unit_step_gathers_kept_rows(k):
    q, kw = _rand(50, 8, 16, 4)
    vw = np.arange(64, dtype=float).reshape(16, 4)
    res = k.unit_step(q, kw, kw, vw, 6, 1, 1)
    assert np.array_equal(res["k_new"], kw[res["keep"]])
    assert np.array_equal(res["v_new"], vw[res["keep"]])
    assert np.array_equal(res["keep"], k.token2chunk_keep(k.window_scores(q, kw), 6, 1, 1))


def pin_step_unit_gqa_and_window(k):
    """step_unit takes the last window_len rows of the unit and the window
    queries of query heads h*G .. h*G+G-1 only (here G = 2, h = 1)."""
    from types import SimpleNamespace
    rng = np.random.default_rng([78, 60])
    hq, hkv, w, d, n = 4, 2, 6, 4, 15
    kc = SimpleNamespace(window_len=w, keep=3, anchors=1, radius=1)
    q = rng.standard_normal((hq, w, d)).astype(np.float32)
    krows = rng.standard_normal((n, d)).astype(np.float32)
    vrows = rng.standard_normal((n, d)).astype(np.float32)
    res = k.step_unit(kc, "f32", hq, hkv, q, krows, vrows, 1)
    rows = np.concatenate([q[2], q[3]]).astype(np.float64)
    s = brute.kara_scores(rows.tolist(), krows[n - w:].astype(np.float64).tolist())
    _close(res["score"], s)
    want = brute.kara_keep(s, 3, 1, 1)
    assert list(res["keep"]) == want
    assert np.array_equal(res["k_new"], krows[n - w:][want])
    assert np.array_equal(res["v_new"], vrows[n - w:][want])


def _bf16_bits(x):
    """bf16 storage of float32 values that bf16 holds exactly (a bf16 is the
    upper half of an IEEE binary32)."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    assert np.all(bits & np.uint32(0xFFFF) == 0), "value not exact in bf16"
    return (bits >> np.uint32(16)).astype(np.uint16)


def pin_decode_bf16_patterns(k):
    """bf16 widening against hand-decoded bit patterns: sign, exponent bias
    127, 7 stored fraction bits, subnormals, infinities."""
    pats = [0x3F80, 0xBF80, 0x4040, 0x3F81, 0xC2F7, 0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x0080]
    want = [1.0, -1.0, 3.0, 1.0 + 2.0 ** -7, -123.5, 0.0, -0.0, 2.0 ** -133, math.inf, -math.inf,
            2.0 ** -126]
    got = k._decode(np.array(pats, dtype=np.uint16), "bf16")
    assert got.dtype == np.float64
    for g, w_, p in zip(got, want, pats):
        assert g == w_ and math.copysign(1.0, g) == math.copysign(1.0, w_), (hex(p), g, w_)


def pin_step_unit_bf16(k):
    """step_unit on bf16 storage: scores from the widened values, kept rows
    returned as the stored bit patterns (here G = 2, h = 0)."""
    from types import SimpleNamespace
    rng = np.random.default_rng([78, 61])
    hq, hkv, w, d, n = 4, 2, 8, 4, 13
    kc = SimpleNamespace(window_len=w, keep=4, anchors=1, radius=1)
    # small multiples of 1/8: exact in bf16
    q = (rng.integers(-16, 17, (hq, w, d)) / 8.0).astype(np.float32)
    krows = (rng.integers(-16, 17, (n, d)) / 8.0).astype(np.float32)
    vrows = (rng.integers(-16, 17, (n, d)) / 8.0).astype(np.float32)
    qb, kb, vb = _bf16_bits(q), _bf16_bits(krows), _bf16_bits(vrows)
    res = k.step_unit(kc, "bf16", hq, hkv, qb, kb, vb, 0)
    rows = np.concatenate([q[0], q[1]]).astype(np.float64)
    s = brute.kara_scores(rows.tolist(), krows[n - w:].astype(np.float64).tolist())
    _close(res["score"], s)
    want = brute.kara_keep(s, 4, 1, 1)
    assert list(res["keep"]) == want
    assert res["k_new"].dtype == np.uint16 and np.array_equal(res["k_new"], kb[n - w:][want])
    assert res["v_new"].dtype == np.uint16 and np.array_equal(res["v_new"], vb[n - w:][want])


ALL_PINS = [v for kk, v in sorted(globals().items()) if kk.startswith("pin_")]
