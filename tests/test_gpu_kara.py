"""rkv_kara_step, the KARA-style sliding-window step, against the KARA oracle
(oracle/kara_oracle.py) on the same seeded inputs: window scores within
1e-3 of the float64 oracle (relative to the unit's largest score), the kept
set equal to the oracle's Token2Chunk rule applied to the kernel's own float32
scores and to the float64 oracle's set except where the oracle's scores tie
within that tolerance at a decision, compacted rows bit-exact, the prefix and
the rows past the new length untouched, FREE_BLOCKS bit-exact, sequences below
the trigger untouched."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import ContigCase, PagedCase, canary_value, log, to_dev, to_host
from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.gpu

TOL = 1e-3


def shape_cfg(spec):
    return B.make_config(spec.num_layers, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         spec.budget, spec.buffer, spec.window, spec.mix_lambda, spec.dtype,
                         spec.layout, spec.block_size)


def run_kara(case, kc, tails, workspace=None, q_host=None):
    spec = case.spec
    W, K = kc.window_len, kc.keep
    if q_host is None:
        q_host = syn.build_queries(spec.with_(window=W))
    q = to_dev(q_host)
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    scores = torch.full((rows * W,), float("nan"), device="cuda")
    keep = torch.full((rows * K,), -7, dtype=torch.int32, device="cuda")
    lens = case.lens0.astype(np.int32).copy()
    tail = np.array(tails, dtype=np.int32)
    counts = np.zeros(spec.num_seqs, np.int32)
    fcap = 0
    if spec.layout == "paged":
        bs = spec.block_size
        fcap = sum(-(-int(n) // bs) - -(-(int(n) - W + K) // bs)
                   for n, t in zip(case.lens0, tails) if n - t >= W)
    fb = torch.full((max(1, fcap),), -9, dtype=torch.int32, device="cuda")
    B.rkv_kara_step(shape_cfg(spec), kc, case.cache, q, spec.num_seqs, lens, tail, scores, keep,
                    fb if spec.layout == "paged" else None, fcap, counts, workspace,
                    0 if workspace is None else workspace.numel())
    torch.cuda.synchronize()
    return SimpleNamespace(q_host=q_host, scores=scores.cpu().numpy().reshape(rows, W),
                           keep=keep.cpu().numpy().reshape(rows, K), lens=lens, tail=tail,
                           counts=counts, fb=fb.cpu().numpy()[:fcap], fcap=fcap)


def decisive_tie(k_or, s, kc, tol):
    """True if the oracle's scores s tie within tol at one of the rule's
    decisions: the last anchor against the next token, or the last filled
    place against the next candidate outside the chunks."""
    order = k_or.rank_order(s)
    m, r, K = kc.anchors, kc.radius, kc.keep
    if 0 < m < len(s) and abs(s[order[m - 1]] - s[order[m]]) <= tol:
        return True
    in_chunk = np.zeros(len(s), bool)
    for a in order[:m]:
        in_chunk[max(0, a - r): a + r + 1] = True
    rest = [j for j in order if not in_chunk[j]]
    left = K - int(in_chunk.sum())
    return 0 < left < len(rest) and abs(s[rest[left - 1]] - s[rest[left]]) <= tol


def check(case, kc, tails, res, units=None, before=None):
    from oracle import kara_oracle as KO
    spec = case.spec
    W, K, G = kc.window_len, kc.keep, spec.group
    trig = [s for s in range(spec.num_seqs) if case.lens0[s] - tails[s] >= W]
    ties = 0
    for s in range(spec.num_seqs):
        n = int(case.lens0[s])
        if s not in trig:
            assert res.lens[s] == n and res.tail[s] == tails[s] and res.counts[s] == 0
            continue
        assert res.lens[s] == n - W + K and res.tail[s] == n - W + K
    todo = units if units is not None else [(s, l, h) for s in trig for l in range(spec.num_layers)
                                             for h in range(spec.num_kv_heads)]
    for (s, l, h) in todo:
        n = int(case.lens0[s])
        t0 = n - W
        row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
        where = f"unit (s={s}, l={l}, h={h}) N={n}"
        krows, vrows = before(s, l, h)
        o = KO.step_unit(kc, spec.dtype, spec.num_q_heads, spec.num_kv_heads, res.q_host[l, s],
                         krows, vrows, h)
        g = res.scores[row].astype(np.float64)
        tol = TOL * np.abs(o["score"]).max()
        err = np.abs(g - o["score"]).max()
        assert err <= tol, f"{where}: score off by {err:.3e} (tol {tol:.3e})"
        kept = res.keep[row].astype(np.int64)
        same = KO.token2chunk_keep(g, K, kc.anchors, kc.radius)
        assert np.array_equal(kept, t0 + same), f"{where}: keep differs from the rule on GPU scores"
        if not np.array_equal(same, o["keep"]):
            assert decisive_tie(KO, o["score"], kc, 2 * tol), f"{where}: keep differs without a tie"
            ties += 1
        gk, gv = case.gpu_rows(s, l, h, n)
        assert np.array_equal(gk[:t0], krows[:t0]) and np.array_equal(gv[:t0], vrows[:t0]), \
            f"{where}: prefix changed"
        assert np.array_equal(gk[t0:t0 + K], krows[t0:][same]), f"{where}: compacted K differs"
        assert np.array_equal(gv[t0:t0 + K], vrows[t0:][same]), f"{where}: compacted V differs"
        moved = t0 + np.flatnonzero(same != np.arange(K))
        untouched = np.setdiff1d(np.arange(t0, n), moved)
        assert np.array_equal(gk[untouched], krows[untouched]), f"{where}: a row past the kept ones changed"
        assert np.array_equal(gv[untouched], vrows[untouched])
    if spec.layout == "paged":
        want = []
        for s in trig:
            n = int(case.lens0[s])
            want += KO.free_blocks(case.bt[s], n, n - W + K, spec.block_size)
        assert list(res.fb) == want
    return ties


def contig_before(case):
    return lambda s, l, h: case.unit_rows(s, l, h)


CONTIG = [
    (syn.config(1).with_(name="kara-llama", seed=71, num_seqs=3, num_layers=2, lens=(1152, 1100, 1200)),
     SimpleNamespace(window_len=128, keep=32, anchors=4, radius=2), (1024, 900, 1100)),
    (syn.config(1).with_(name="kara-d64", seed=72, num_seqs=3, num_layers=2, num_q_heads=16,
                         num_kv_heads=2, head_dim=64, lens=(300, 200, 250)),
     SimpleNamespace(window_len=64, keep=16, anchors=2, radius=1), (236, 100, 200)),
    # head_dim 64 at the other two window lengths (2 and 8 key blocks in each
    # strided LDS read of the window keys)
    (syn.config(1).with_(name="kara-d64-w32", seed=78, num_seqs=3, num_layers=2, num_q_heads=8,
                         num_kv_heads=2, head_dim=64, lens=(300, 200, 250)),
     SimpleNamespace(window_len=32, keep=12, anchors=2, radius=2), (236, 100, 230)),
    (syn.config(1).with_(name="kara-d64-w128", seed=79, num_seqs=3, num_layers=2, num_q_heads=16,
                         num_kv_heads=2, head_dim=64, lens=(400, 300, 260)),
     SimpleNamespace(window_len=128, keep=40, anchors=3, radius=2), (200, 172, 200)),
    # G 1 at head_dim 64: two query tiles, so two waves score none (their V
    # rows are copied before the tile loop) while the keys go through LDS
    (syn.config(1).with_(name="kara-d64-w32-g1", seed=80, num_seqs=2, num_layers=2, num_q_heads=4,
                         num_kv_heads=4, head_dim=64, lens=(160, 90)),
     SimpleNamespace(window_len=32, keep=10, anchors=1, radius=3), (100, 40)),
    (syn.config(1).with_(name="kara-w32-keep-all", seed=73, num_seqs=2, num_layers=2, num_q_heads=8,
                         num_kv_heads=8, lens=(96, 40)),
     SimpleNamespace(window_len=32, keep=32, anchors=0, radius=0), (64, 0)),
    (syn.config(1).with_(name="kara-w32-keep-one", seed=74, num_seqs=2, num_layers=1, lens=(33, 70)),
     SimpleNamespace(window_len=32, keep=1, anchors=1, radius=0), (0, 30)),
    (syn.config(1).with_(name="kara-wide-chunks", seed=75, num_seqs=1, num_layers=3, num_q_heads=64,
                         num_kv_heads=8, lens=(700,), dup_mode="runs", dup_frac=0.4),
     SimpleNamespace(window_len=128, keep=60, anchors=3, radius=9), (500,)),
]


@pytest.mark.parametrize("spec,kc,tails", CONTIG, ids=[c[0].name for c in CONTIG])
def test_kara_contiguous(spec, kc, tails):
    log(f"kara: {spec.name}")
    case = ContigCase(spec)
    before = {(s, l, h): case.unit_rows(s, l, h) for s in range(spec.num_seqs)
              for l in range(spec.num_layers) for h in range(spec.num_kv_heads)}
    res = run_kara(case, B.rkv_kara_config(kc.window_len, kc.keep, kc.anchors, kc.radius), tails)
    ties = check(case, kc, tails, res, before=lambda s, l, h: (before[(s, l, h)][0].copy(),
                                                                 before[(s, l, h)][1].copy()))
    log(f"kara: {spec.name}: {ties} units decided by an oracle near-tie")
    # sequences below the trigger: cache rows and outputs untouched
    W = kc.window_len
    for s in range(spec.num_seqs):
        if case.lens0[s] - tails[s] >= W:
            continue
        for l in range(spec.num_layers):
            for h in range(spec.num_kv_heads):
                row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
                assert np.isnan(res.scores[row]).all() and (res.keep[row] == -7).all()
                n = int(case.lens0[s])
                gk, gv = case.gpu_rows(s, l, h, n)
                assert np.array_equal(gk, before[(s, l, h)][0]) and np.array_equal(gv, before[(s, l, h)][1])


PAGED = [
    (syn.config(3).with_(name="kara-paged", seed=76, num_seqs=3, num_layers=2, budget=1024,
                         buffer=128, num_blocks=400, lens=(1152, 1000, 777)),
     SimpleNamespace(window_len=128, keep=32, anchors=4, radius=2), (1024, 872, 700)),
    (syn.config(3).with_(name="kara-paged-bs32", seed=77, num_seqs=2, num_layers=2, budget=256,
                         buffer=32, block_size=32, num_blocks=64, lens=(300, 150)),
     SimpleNamespace(window_len=64, keep=20, anchors=2, radius=2), (200, 86)),
]


@pytest.mark.parametrize("spec,kc,tails", PAGED, ids=[c[0].name for c in PAGED])
def test_kara_paged(spec, kc, tails):
    log(f"kara: {spec.name}")
    case = PagedCase(spec)
    k_before, v_before = case.k.clone(), case.v.clone()
    before = {(s, l, h): case.unit_rows(s, l, h) for s in range(spec.num_seqs)
              for l in range(spec.num_layers) for h in range(spec.num_kv_heads)}
    res = run_kara(case, B.rkv_kara_config(kc.window_len, kc.keep, kc.anchors, kc.radius), tails)
    check(case, kc, tails, res, before=lambda s, l, h: before[(s, l, h)])
    # blocks no triggered sequence references are untouched (canary included)
    used = set()
    for s in range(spec.num_seqs):
        used |= set(int(b) for b in case.bt[s][: -(-int(case.lens0[s]) // spec.block_size)])
    free_idx = torch.tensor(sorted(set(range(spec.num_blocks)) - used), device="cuda")
    assert torch.equal(case.k.index_select(1, free_idx), k_before.index_select(1, free_idx))
    assert torch.equal(case.v.index_select(1, free_idx), v_before.index_select(1, free_idx))


def test_kara_llama8b_full_batch():
    """The Llama-8B-shaped batch the benchmark times: 32 layers x 8 kv heads,
    N 1152 with the last 128 tokens as the window, keep 32 (4 anchors of
    radius 2): all 256 units against the oracle."""
    spec = syn.config(1)
    kc = SimpleNamespace(window_len=128, keep=32, anchors=4, radius=2)
    case = ContigCase(spec)
    res = run_kara(case, B.rkv_kara_config(128, 32, 4, 2), (1024,))
    ties = check(case, kc, (1024,), res, before=contig_before_from_host(case))
    log(f"kara full batch: {ties} of 256 units decided by an oracle near-tie")


@pytest.mark.parametrize("mode", ["zero-queries", "two-key-values"])
def test_kara_exact_ties(mode):
    """Scores that tie exactly, where only the position order decides.
    zero-queries: every window token gets weight 1/W from every row, so all
    scores are equal and the rule keeps the window's first `keep` tokens (a
    reversed tie order would keep the last ones).  two-key-values: the window
    keys alternate between two vectors, so the scores take two values and
    each group is ranked by position; the anchors' chunks then make rows
    move.  Both against the oracle, whose float64 scores tie the same way."""
    spec = syn.config(1).with_(name=f"kara-ties-{mode}", seed=78, num_seqs=2, num_layers=2,
                               num_q_heads=8, num_kv_heads=2, lens=(400, 300))
    kc = SimpleNamespace(window_len=64, keep=20, anchors=2, radius=3)
    W, tails = kc.window_len, (336, 236)
    case = ContigCase(spec)
    q_host = None
    if mode == "zero-queries":
        q_host = np.zeros_like(syn.build_queries(spec.with_(window=W)))
    else:
        for s in range(spec.num_seqs):
            t0 = int(case.lens0[s]) - W
            win = case.k_host[:, s, :, t0:t0 + W]
            win[:, :, 0::2] = win[:, :, :1].copy()
            win[:, :, 1::2] = win[:, :, 1:2].copy()
        case.k.copy_(to_dev(case.k_host))
    before = {(s, l, h): (case.unit_rows(s, l, h)[0].copy(), case.unit_rows(s, l, h)[1].copy())
              for s in range(spec.num_seqs) for l in range(spec.num_layers)
              for h in range(spec.num_kv_heads)}
    res = run_kara(case, B.rkv_kara_config(W, kc.keep, kc.anchors, kc.radius), tails, q_host=q_host)
    ties = check(case, kc, tails, res, before=lambda s, l, h: before[(s, l, h)])
    assert ties == 0, "exact ties are decided by position on both sides"
    if mode == "zero-queries":
        for s in range(spec.num_seqs):
            t0 = int(case.lens0[s]) - W
            for l in range(spec.num_layers):
                for h in range(spec.num_kv_heads):
                    row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
                    assert np.all(res.scores[row] == res.scores[row][0])
                    assert np.array_equal(res.keep[row], t0 + np.arange(kc.keep))
    else:
        moved = sum(int((res.keep[r] != res.keep[r][0] + np.arange(kc.keep)).any())
                    for r in range(res.keep.shape[0]))
        assert moved > 0, "the two-valued scores should make some kept rows move"


def contig_before_from_host(case):
    # the host copies of the inputs (case.k_host) are never written
    return lambda s, l, h: case.unit_rows(s, l, h)


def test_kara_bad_block_id_and_status():
    """With the block check on, an id past the declared pool (inside the
    allocation) stops the step: nothing written, the status reported."""
    spec = PAGED[0][0].with_(name="kara-bad-id", seed=78)
    case = PagedCase(spec)
    nb = spec.num_blocks
    L, _, hk, bs, d = case.k.shape
    per = hk * bs * d
    big_k = torch.full((L, (nb + 8) * per), canary_value(spec), dtype=case.k.dtype, device="cuda")
    big_v = big_k.clone()
    big_k[:, :nb * per] = case.k.reshape(L, -1)
    big_v[:, :nb * per] = case.v.reshape(L, -1)
    bad = case.bt.copy()
    bad[0, 5] = nb + 3
    bt_dev = torch.from_numpy(bad).cuda()
    cache = B.make_cache(big_k, big_v, num_blocks=nb, block_table=bt_dev,
                         max_blocks_per_seq=bad.shape[1], layer_stride=(nb + 8) * per)
    cfg = shape_cfg(spec)
    cfg.check_block_table = 1
    snap = (big_k.clone(), big_v.clone())
    W, K = 128, 32
    q = to_dev(syn.build_queries(spec.with_(window=W)))
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    scores = torch.full((rows * W,), float("nan"), device="cuda")
    keep = torch.full((rows * K,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    lens = case.lens0.astype(np.int32).copy()
    tail = np.array(PAGED[0][2], np.int32)
    fb = torch.full((64,), -9, dtype=torch.int32, device="cuda")
    B.rkv_kara_step(cfg, B.rkv_kara_config(W, K, 4, 2), cache, q, spec.num_seqs, lens, tail, scores,
                    keep, fb, 64, None, ws, 256)
    assert B.rkv_device_status(ws) == B.RKV_DEVICE_BAD_BLOCK_ID
    assert torch.equal(big_k, snap[0]) and torch.equal(big_v, snap[1])
    assert bool((keep == -7).all()) and bool(torch.isnan(scores).all()) and bool((fb == -9).all())
