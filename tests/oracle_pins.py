"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin takes the oracle module as an argument, so the mutation test can run
the same pins against deliberately broken copies of it.  The pins use:
hand-derived worked examples (tests/golden/hand_examples.json), defaults the
pages print (tests/golden/page_defaults.json), invariants and closed forms of
the mathematics, special cases that reduce to a library routine, and the
scalar brute force in oracle/brute.py on tiny inputs.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))


def golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.abs(a - b) <= tol * np.maximum(1.0, np.abs(b))), (a, b)


def _rand_case(seed, n, d, rows, dup=0):
    rng = np.random.default_rng([77, seed])
    k = rng.standard_normal((n, d)) + rng.standard_normal(d) * 0.5
    for _ in range(dup):
        a, b = sorted(rng.choice(n, 2, replace=False))
        k[b] = k[a] + 0.01 * rng.standard_normal(d)
    q = rng.standard_normal((rows, d))
    return q, k


# ------------------------------------------------------------- worked examples

def pin_golden_importance(o):
    for ex in golden("hand_examples.json")["importance"]:
        _close(o.importance(np.array(ex["q"]), np.array(ex["k"])), ex["expect"])


def pin_golden_redundancy(o):
    for ex in golden("hand_examples.json")["redundancy"]:
        _close(o.redundancy(np.array(ex["k"])), ex["expect"])


def pin_golden_step(o):
    for ex in golden("hand_examples.json")["step"]:
        q, k = np.array(ex["q"]), np.array(ex["k"])
        r = o.unit_step(q, k, k, k, ex["budget"], ex["window"], ex["lam"])
        _close(r["score"], ex["expect_S"])
        assert list(r["keep"]) == ex["expect_keep"], r["keep"]
        _close(r["k_new"], ex["expect_k_new"])


def pin_golden_select(o):
    for ex in golden("hand_examples.json")["select"]:
        got = o.select_keep(np.array(ex["scores"]), ex["n"], ex["budget"], ex["window"])
        assert list(got) == ex["expect"], (ex["name"], got)


def pin_golden_select_shared(o):
    for ex in golden("hand_examples.json")["select_shared"]:
        got = o.select_keep_shared(np.array(ex["scores"]), ex["n"], ex["budget"], ex["window"])
        assert list(got) == ex["expect"], (ex["name"], got)


def pin_golden_free_blocks(o):
    for ex in golden("hand_examples.json")["free_blocks"]:
        got = o.free_blocks(ex["bt_row"], ex["n"], ex["budget"], ex["block_size"])
        assert list(got) == ex["expect"], (ex["name"], got)


def pin_golden_trigger(o):
    for ex in golden("hand_examples.json")["trigger"]:
        assert bool(o.is_triggered(ex["n"], ex["budget"], ex["buffer"])) == ex["expect"], ex


# ------------------------------------------------------------- storage decode

def _bf16_by_struct(bits):
    """bf16 bits -> float through the standard library: the 16 bits are the
    top half of an IEEE-754 binary32 (sign, 8-bit exponent, 7 mantissa bits)."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def pin_decode_bf16_known_patterns(o):
    """Fixed bf16 patterns with values known from the binary32 format."""
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x8000: -0.0, 0x0000: 0.0,
             0x4049: 3.140625, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x0080: 2.0 ** -126,
             0xBF40: -0.75, 0x3C00: 2.0 ** -7, 0x7F80: math.inf, 0xFF80: -math.inf}
    bits = np.array(list(cases), dtype=np.uint16)
    got = o.decode(bits, "bf16")
    assert got.dtype == np.float64
    for b, g in zip(cases, got):
        want = cases[b]
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), (hex(b), g, want)
    with np.errstate(invalid="ignore"):
        assert np.isnan(o.decode(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")).all()


def pin_decode_bf16_random_patterns(o):
    """Every finite random bf16 pattern decodes to torch's bfloat16 -> float64
    widening and to the struct-level reading of the format; shapes are kept."""
    import torch
    rng = np.random.default_rng([77, 4])
    bits = rng.integers(0, 1 << 16, size=(64, 33), dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    got = o.decode(bits, "bf16")
    assert got.shape == bits.shape
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[finite], ref[finite])
    for b in bits.ravel()[:300]:
        if (int(b) & 0x7F80) != 0x7F80:
            assert o.decode(np.array([b], dtype=np.uint16), "bf16")[0] == _bf16_by_struct(b)


def pin_decode_f32(o):
    """float32 storage widens exactly: values from their binary32 bit patterns
    (read by struct), subnormals and signed zero included."""
    rng = np.random.default_rng([77, 5])
    pats = [0x3F800000, 0xC0000000, 0x00000001, 0x80000000, 0x007FFFFF, 0x7F7FFFFF, 0x3EAAAAAB]
    pats += [int(x) for x in rng.integers(0, 0x7F000000, size=100)]
    vals = [struct.unpack("<f", struct.pack("<I", p))[0] for p in pats]
    arr = np.array(pats, dtype=np.uint32).view(np.float32)
    got = o.decode(arr, "f32")
    assert got.dtype == np.float64
    for g, want in zip(got, vals):
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want)


def pin_step_unit_gqa(o):
    """step_unit, the per-unit entry the GPU comparisons use: with G = 3 query
    heads per KV head, each KV head h (h = 0, 1, 2) is scored from query heads
    3h .. 3h+2 only.  The expected values come from the scalar brute force on
    rows sliced and decoded here by the standard library, and compaction
    returns the stored bits of the kept rows."""
    import torch
    from types import SimpleNamespace
    rng = np.random.default_rng([77, 6])
    hkv, group, w, d, n = 3, 3, 2, 8, 24
    spec = SimpleNamespace(num_q_heads=hkv * group, num_kv_heads=hkv, dtype="bf16",
                           budget=16, window=w, mix_lambda=0.3)

    def bf16_bits(x):
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)

    q_sl = bf16_bits(rng.standard_normal((hkv * group, w, d)))
    for h in range(hkv):
        k_rows = bf16_bits(rng.standard_normal((n, d)) + rng.standard_normal(d))
        v_rows = bf16_bits(rng.standard_normal((n, d)))
        q_rows = [[_bf16_by_struct(b) for b in q_sl[h * group + g, r]]
                  for g in range(group) for r in range(w)]
        keys = [[_bf16_by_struct(b) for b in row] for row in k_rows]
        bi, br, bs, bkeep = brute.unit(q_rows, keys, spec.mix_lambda, spec.budget, w)
        got = o.step_unit(spec, q_sl, k_rows, v_rows, h)
        _close(got["imp"], bi)
        _close(got["red"], br)
        _close(got["score"], bs)
        assert list(got["keep"]) == bkeep, h
        assert got["k_new"].dtype == np.uint16 and np.array_equal(got["k_new"], k_rows[bkeep])
        assert np.array_equal(got["v_new"], v_rows[bkeep])


# ------------------------------------------------------------- invariants

def pin_attention_rows_sum_to_one(o):
    """Each softmax row sums to 1, so the row mean I sums to 1 over the keys."""
    for seed, (n, d, rows) in enumerate([(40, 16, 8), (160, 64, 32), (33, 8, 56)]):
        q, k = _rand_case(seed, n, d, rows)
        imp = o.importance(q, k)
        assert abs(imp.sum() - 1.0) < 1e-12
        assert np.all(imp > 0)


def pin_zero_query_uniform(o):
    for n in (2, 17, 160):
        _, k = _rand_case(n, n, 16, 1)
        imp = o.importance(np.zeros((8, 16)), k)
        assert np.all(imp == 1.0 / n) or np.allclose(imp, 1.0 / n, rtol=1e-15, atol=0)


def pin_importance_scale(o):
    """Scale 1/sqrt(d): for two orthonormal keys and q = a*e0, the weight of
    key 0 is 1/(1 + exp(-a/sqrt(d))) whatever the padding dimension d."""
    for d in (2, 16, 128):
        k = np.zeros((2, d))
        k[0, 0] = 1.0
        k[1, 1] = 1.0
        a = 3.0
        q = np.zeros((1, d))
        q[0, 0] = a
        imp = o.importance(q, k)
        _close(imp[0], 1.0 / (1.0 + math.exp(-a / math.sqrt(d))))


def pin_importance_shift_invariant(o):
    """A query whose dot product is the same with every key (it is orthogonal
    to all key differences) gives uniform weights, whatever that value is."""
    d = 8
    base = np.zeros(d)
    base[0] = 2.0
    k = np.tile(base, (5, 1))
    k[:, 1:] = np.random.default_rng(3).standard_normal((5, d - 1))
    q = np.zeros((3, d))
    q[:, 0] = [1.0, -4.0, 9.0]          # q.k_j is the same for every j
    _close(o.importance(q, k), np.full(5, 0.2))


def pin_gram_diagonal_is_one(o):
    _, k = _rand_case(5, 50, 32, 1)
    c = o.cosine_gram(k)
    _close(np.diag(c), np.ones(50))
    _close(c, c.T)
    assert np.all(np.abs(c) <= 1.0 + 1e-12)


def pin_redundancy_rank_one_closed_form(o):
    """Sum_{k != j} khat_j . khat_k = khat_j . (sum_k khat_k) - 1, computed here
    without forming the Gram matrix."""
    for seed, (n, d) in enumerate([(7, 3), (160, 64), (300, 128)]):
        _, k = _rand_case(seed + 10, n, d, 1, dup=n // 5)
        khat = k / np.linalg.norm(k, axis=1, keepdims=True)
        total = khat.sum(axis=0)
        expect = (khat @ total - 1.0) / (n - 1)
        _close(o.redundancy(k), expect, tol=1e-12)


def pin_redundancy_rowwise_equals_gram(o):
    """The one-row-at-a-time redundancy (for long caches) equals the Gram-based
    one, zero keys and duplicates included."""
    for seed in range(4):
        _, k = _rand_case(500 + seed, 37, 16, 1, dup=3)
        k[5] = 0.0
        idx = [0, 5, 17, 36]
        _close(o.redundancy_at(k, idx), o.redundancy(k)[idx])
        _close(o.redundancy_at(k, range(37)), o.redundancy(k))


def pin_redundancy_scale_invariant(o):
    """Cosine ignores each key's length: scaling keys by different positive
    factors leaves R unchanged."""
    _, k = _rand_case(21, 64, 16, 1)
    c = np.exp(np.random.default_rng(4).uniform(-3, 3, size=(64, 1)))
    _close(o.redundancy(k * c), o.redundancy(k), tol=1e-12)


def pin_exact_duplicates(o):
    """k_b = 2 k_a: their cosine is 1 (the largest possible entry) and R_a = R_b."""
    _, k = _rand_case(22, 40, 16, 1)
    k[31] = 2.0 * k[9]
    c = o.cosine_gram(k)
    _close(c[9, 31], 1.0)
    off = c - np.diag(np.diag(c))
    assert c[9, 31] >= off.max() - 1e-15
    r = o.redundancy(k)
    _close(r[9], r[31], tol=1e-14)


def pin_constructed_duplicate_is_maximal_and_evicted(o):
    """Orthonormal e1..e5 plus a copy of e1: the copied pair has redundancy
    1/(N-1), every other key 0.  With lam = 0 and one eviction, the later copy
    goes (equal scores keep the lower position)."""
    d = 8
    eye = np.eye(d)
    k = np.stack([eye[0], eye[1], eye[2], eye[3], eye[0], eye[4]])
    n = 6
    r = o.redundancy(k)
    _close(r, [0.2, 0, 0, 0, 0.2, 0])
    _, red, s = o.score_unit(np.zeros((1, d)), k, 0.0)
    keep = o.select_keep(s, n, budget=5, window=1)
    assert list(keep) == [0, 1, 2, 3, 5], keep


def pin_lambda_one_is_attention_topk(o):
    """lam = 1: the keep set is the top-(B - w) candidates by window attention
    alone -- here computed with torch's softmax and a stable sort."""
    import torch
    for seed, (n, d, rows, b, w) in enumerate([(160, 64, 32, 128, 8), (90, 16, 8, 50, 4)]):
        q, k = _rand_case(seed + 30, n, d, rows)
        logits = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(d)
        p = torch.softmax(logits, dim=1).mean(dim=0)
        cand = p[: n - w]
        order = torch.sort(cand, descending=True, stable=True).indices[: b - w]
        expect = sorted(order.tolist()) + list(range(n - w, n))
        _, _, s = o.score_unit(q, k, 1.0)
        assert list(o.select_keep(s, n, b, w)) == expect


def pin_lambda_zero_is_low_redundancy(o):
    """lam = 0: candidates ranked by redundancy ascending."""
    q, k = _rand_case(40, 120, 32, 16, dup=30)
    imp, red, s = o.score_unit(q, k, 0.0)
    _close(s, -red)
    n, b, w = 120, 70, 8
    order = np.argsort(red[: n - w], kind="stable")[: b - w]
    assert list(o.select_keep(s, n, b, w)) == sorted(order.tolist()) + list(range(n - w, n))


def pin_mix_is_affine(o):
    imp = np.array([0.1, 0.5, 0.4])
    red = np.array([0.3, -0.2, 0.9])
    for lam in (0.0, 0.05, 0.1, 0.2, 1.0):
        _close(o.mixed_score(imp, red, lam), lam * imp - (1 - lam) * red)
    # larger importance, same redundancy -> larger score; larger redundancy -> smaller
    s = o.mixed_score(np.array([0.2, 0.3, 0.2]), np.array([0.1, 0.1, 0.2]), 0.1)
    assert s[1] > s[0] > s[2]


def pin_window_always_kept(o):
    rng = np.random.default_rng(8)
    for n, b, w in [(160, 128, 8), (40, 9, 8), (1152, 1024, 8)]:
        s = rng.standard_normal(n)
        s[n - w:] = -1e9            # the window scores worst of all
        keep = o.select_keep(s, n, b, w)
        assert len(keep) == b
        assert np.all(np.diff(keep) > 0)
        assert set(range(n - w, n)) <= set(keep.tolist())
        assert keep.min() >= 0 and keep.max() < n


def pin_select_permutation_equivariant(o):
    """Permuting candidate keys permutes their scores and the kept set (tie-free)."""
    q, k = _rand_case(50, 100, 16, 8)
    n, b, w = 100, 60, 4
    _, _, s = o.score_unit(q, k, 0.1)
    keep = set(o.select_keep(s, n, b, w).tolist())
    perm = np.random.default_rng(9).permutation(n - w)
    full = np.concatenate([perm, np.arange(n - w, n)])
    _, _, s2 = o.score_unit(q, k[full], 0.1)
    _close(s2, s[full], tol=1e-9)
    keep2 = o.select_keep(s2, n, b, w)
    assert {int(full[i]) for i in keep2} == keep


def pin_gqa_grouping_matches_repeat_interleave(o):
    """GQA: kv head h serves the query heads that torch.repeat_interleave maps
    onto it when the kv heads are expanded to the query-head count (the usual
    key/value expansion of grouped-query attention)."""
    import torch
    hq, hkv, w, d = 8, 2, 3, 4
    group = hq // hkv
    q = np.arange(hq * w * d, dtype=np.float64).reshape(hq, w, d)
    owner = torch.repeat_interleave(torch.arange(hkv), group).numpy()
    for h in range(hkv):
        rows = o.q_group(q, h, group)
        expect = q[owner == h].reshape(-1, d)
        assert rows.shape == expect.shape and np.array_equal(rows, expect)


def pin_compaction_is_gather(o):
    rows = np.arange(60, dtype=np.float64).reshape(20, 3)
    keep = np.array([0, 2, 3, 7, 18, 19])
    got = o.compact_rows(rows, keep)
    assert got.shape == (6, 3)
    for i, j in enumerate(keep):
        assert np.array_equal(got[i], rows[j])


def pin_free_blocks_vs_brute(o):
    rng = np.random.default_rng(12)
    for bs in (16, 32):
        for _ in range(50):
            n = int(rng.integers(2, 600))
            b = int(rng.integers(1, n + 1))
            row = rng.permutation(1000)[: -(-n // bs)]
            assert list(o.free_blocks(row, n, b, bs)) == brute.free_blocks(row, n, b, bs)


# ------------------------------------------------------------- brute force

def pin_brute_force_agreement(o):
    """Scalar loops vs the oracle on tiny random cases, including exact ties."""
    cases = [(12, 4, 3, 8, 2, 0.1), (40, 8, 8, 30, 4, 0.1), (64, 16, 32, 48, 8, 0.0),
             (30, 6, 12, 20, 3, 1.0)]
    for seed, (n, d, rows, b, w, lam) in enumerate(cases):
        q, k = _rand_case(seed + 60, n, d, rows, dup=n // 5)
        if seed == 1:
            k[7] = k[3]                 # exact tie in both scores
        imp, red, s = o.score_unit(q, k, lam)
        bi, br, bsc, bkeep = brute.unit(q.tolist(), k.tolist(), lam, b, w)
        _close(imp, bi)
        _close(red, br)
        _close(s, bsc)
        keep = o.select_keep(s, n, b, w)
        assert list(keep) == bkeep
        assert np.array_equal(o.compact_rows(k, keep), np.array(brute.compact(k.tolist(), bkeep)))


def pin_brute_force_tiny_config(o, spec=None):
    """The whole tiny fp32 workload (one unit, N=160, d=64, 32 window rows)
    against the scalar loops."""
    import rkv_synth as syn
    spec = syn.config(0) if spec is None else spec
    n = int(syn.seq_lens(spec)[0])
    kst = syn.keys(spec, 0, 0)[0]
    q = o.decode(syn.queries(spec, 0, 0), spec.dtype).reshape(-1, spec.head_dim)
    k = o.decode(kst, spec.dtype)
    imp, red, s = o.score_unit(q, k, spec.mix_lambda)
    bi, br, bsc, bkeep = brute.unit(q.tolist(), k.tolist(), spec.mix_lambda, spec.budget, spec.window)
    _close(imp, bi)
    _close(red, br)
    _close(s, bsc)
    assert list(o.select_keep(s, n, spec.budget, spec.window)) == bkeep


def pin_shared_selection_special_cases(o):
    """Head-shared selection: one KV head is the per-head rule; identical
    heads (4 of them, so the sum is exact) select what each would alone; the
    heads' order does not matter (integer-valued scores: exact sums); scalar
    brute force agrees on random cases."""
    rng = np.random.default_rng([77, 900])
    for trial in range(20):
        n = int(rng.integers(6, 40))
        window = int(rng.integers(1, 4))
        budget = int(rng.integers(window + 1, n + 1))
        s = rng.standard_normal(n)
        assert list(o.select_keep_shared(s[None, :], n, budget, window)) == \
            list(o.select_keep(s, n, budget, window))
        assert list(o.select_keep_shared(np.stack([s] * 4), n, budget, window)) == \
            list(o.select_keep(s, n, budget, window))
        hs = rng.integers(-20, 20, size=(3, n)).astype(np.float64)
        ref = list(o.select_keep_shared(hs, n, budget, window))
        assert list(o.select_keep_shared(hs[::-1].copy(), n, budget, window)) == ref
        assert ref == brute.select_keep_shared(hs.tolist(), n, budget, window)
        assert ref[-window:] == list(range(n - window, n))


def pin_shared_layer_step(o):
    """The head-shared layer step: every head's scores equal its per-head
    unit scores, every head gets the same keep set (the rule applied to the
    summed scores), and compaction gathers each head's own rows."""
    rng = np.random.default_rng([77, 901])
    heads, n, d, rows = 3, 24, 8, 4
    qs = [rng.standard_normal((rows, d)) for _ in range(heads)]
    ks = [rng.standard_normal((n, d)) for _ in range(heads)]
    vs = [rng.standard_normal((n, d)) for _ in range(heads)]
    res = o.layer_step_shared(qs, ks, ks, vs, 16, 3, 0.3)
    per = [o.unit_step(q, k, k, v, 16, 3, 0.3) for q, k, v in zip(qs, ks, vs)]
    total = brute.select_keep_shared([list(p["score"]) for p in per], n, 16, 3)
    for h in range(heads):
        _close(res[h]["score"], per[h]["score"])
        assert list(res[h]["keep"]) == total
        _close(res[h]["v_new"], vs[h][np.array(total)])
        _close(res[h]["k_new"], ks[h][np.array(total)])


def pin_window_ring_holds_last_queries(o):
    """After any window consecutive decode steps the ring holds exactly the
    last window queries, query t in slot t mod window; layers outside the
    call are untouched."""
    rng = np.random.default_rng([77, 90])
    L, S, Hq, w, d = 3, 3, 2, 4, 3
    start = [0, 5, 13]
    ring = np.full((L, S, Hq, w, d), -1.0)
    history = []
    for t in range(7):
        q = rng.standard_normal((2, S, Hq, d))
        steps = [s0 + t for s0 in start]
        ring = o.window_store(ring, q, 1, steps, w)
        history.append((steps, q))
    assert np.all(ring[0] == -1.0), "layer 0 was not part of the calls"
    for s in range(S):
        for h in range(Hq):
            for li in range(2):
                want = {tuple(q[li, s, h]) for _, q in history[-w:]}
                got = {tuple(ring[1 + li, s, h, j]) for j in range(w)}
                assert got == want
            for steps, q in history[-w:]:
                assert np.array_equal(ring[1:, s, h, steps[s] % w], q[:, s, h])


def pin_importance_ignores_window_row_order(o):
    """The ring keeps the window queries in rotated order; importance is a
    mean over the rows, so any order of them gives the same result."""
    q, k = _rand_case(91, 40, 8, 12)
    perm = np.random.default_rng([77, 91]).permutation(q.shape[0])
    _close(o.importance(q[perm], k), o.importance(q, k), tol=1e-13)
    roll = np.roll(q.reshape(3, 4, 8), 1, axis=1).reshape(12, 8)   # a rotated ring per head
    _close(o.importance(roll, k), o.importance(q, k), tol=1e-13)


def pin_page_defaults(o):
    """The workloads use the pages' default knobs."""
    import rkv_synth as syn
    g = golden("page_defaults.json")
    c1 = syn.config(1)
    assert (c1.budget, c1.window, c1.mix_lambda, c1.buffer) == (
        g["kv_budget"], g["window_size"], g["mix_lambda"], g["divide_length"])
    shape = g["llama8b_shape"]
    assert (c1.num_layers, c1.num_q_heads, c1.num_kv_heads, c1.head_dim) == (
        shape["num_layers"], shape["num_q_heads"], shape["num_kv_heads"], shape["head_dim"])
    lo, hi = g["lambda_tuning_range"]
    for spec in syn.CONFIGS:
        assert spec.window == g["window_size"]
        assert lo <= spec.mix_lambda <= hi
        if spec.layout == "paged":
            assert spec.block_size in g["paged_block_sizes"]
    # trigger at budget + divide_length
    assert o.is_triggered(1152, c1.budget, c1.buffer)
    assert not o.is_triggered(1151, c1.budget, c1.buffer)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
