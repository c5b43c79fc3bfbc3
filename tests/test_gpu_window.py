"""GPU parity of rkv_window_store (the window-query ring of the decode loop)
against the oracle's window_store, through the C ABI: the ring bit-exact
after every step (bf16 and fp32, a subset of layers, per-sequence step
counters that start apart, negative counters), the scores of a cache scored
from the ring within tolerance of the oracle's on the chronological window,
and the store captured in a HIP graph that also advances the counters."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import TOL, ContigCase, config_of, log, to_dev, to_host
from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.gpu


def step_queries(spec, rng, count):
    """Random queries of one decode step in storage dtype: (count, S, Hq, d)."""
    x = rng.standard_normal((count, spec.num_seqs, spec.num_q_heads, spec.head_dim)).astype(np.float32)
    if spec.dtype == "bf16":
        return syn.to_bf16_bits(x)
    return x


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_ring_matches_oracle_every_step(dtype, d):
    from oracle import rkv_oracle as O
    spec = syn.config(1).with_(name=f"ring-{dtype}", seed=60, dtype=dtype, head_dim=d, num_seqs=3,
                               num_layers=3, num_q_heads=8, num_kv_heads=2, window=4,
                               budget=64, buffer=16, lens=(80, 80, 80))
    cfg = config_of(spec)
    rng = np.random.default_rng([60, d])
    shape = (spec.num_layers, spec.num_seqs, spec.num_q_heads, spec.window, spec.head_dim)
    ring_h = np.zeros(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    ring = to_dev(ring_h)
    steps_h = np.array([0, 7, -3], dtype=np.int32)       # counters that start apart (and below 0)
    for t in range(11):
        q = step_queries(spec, rng, 2)
        steps = torch.from_numpy(steps_h + t).cuda()
        B.rkv_window_store(cfg, 1, 2, to_dev(q), spec.num_seqs, steps, ring)   # layers 1 and 2
        ring_h = O.window_store(ring_h, q, 1, steps_h + t, spec.window)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(ring, dtype), ring_h), f"ring differs after step {t}"
    assert np.all(to_host(ring, dtype)[0] == 0), "layer 0 written"
    log(f"ring {dtype} d{d}: 11 steps bit-exact against the oracle")


def test_scores_from_ring_match_chronological_window():
    """A decode loop: the ring filled over window + 3 steps, then rkv_score
    reads it; importance and scores match the oracle on the last window
    queries in step order."""
    from oracle import rkv_oracle as O
    spec = syn.config(1).with_(name="ring-score", seed=61, num_seqs=2, num_layers=2, num_q_heads=8,
                               num_kv_heads=2, window=8, budget=200, buffer=40, lens=(300, 257))
    case = ContigCase(spec)
    cfg = config_of(spec)
    rng = np.random.default_rng([61])
    ring = torch.zeros_like(case.q)
    hist = []
    start = np.array([5, 12], dtype=np.int32)
    for t in range(spec.window + 3):
        q = step_queries(spec, rng, spec.num_layers)
        B.rkv_window_store(cfg, 0, spec.num_layers, to_dev(q), spec.num_seqs,
                           torch.from_numpy(start + t).cuda(), ring)
        hist.append(q)
    chrono = np.stack(hist[-spec.window:], axis=3)        # (L, S, Hq, w, d), oldest first
    n = int(case.lens0.max())
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    scores = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    imp = torch.empty_like(scores)
    red = torch.empty_like(scores)
    ws = torch.empty(max(256, B.rkv_workspace_size(cfg, spec.num_seqs, n)), dtype=torch.uint8,
                     device="cuda")
    B.rkv_score(cfg, case.cache, ring, spec.num_seqs, case.lens0.astype(np.int32), scores, n, imp,
                red, ws, ws.numel())
    torch.cuda.synchronize()
    group = spec.num_q_heads // spec.num_kv_heads
    for s in range(spec.num_seqs):
        ns = int(case.lens0[s])
        for l in range(spec.num_layers):
            for h in range(spec.num_kv_heads):
                k = O.decode(case.unit_rows(s, l, h)[0], spec.dtype)
                qr = O.decode(O.q_group(chrono[l, s], h, group), spec.dtype)
                want_i = O.importance(qr, k)
                want_s = O.mixed_score(want_i, O.redundancy(k), spec.mix_lambda)
                row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
                gi = imp[row, :ns].cpu().numpy().astype(np.float64)
                gs = scores[row, :ns].cpu().numpy().astype(np.float64)
                assert np.all(np.abs(gi - want_i) <= TOL * want_i), f"importance ({s},{l},{h})"
                assert np.abs(gs - want_s).max() <= TOL * np.abs(want_s).max(), f"score ({s},{l},{h})"
    log("scores from the ring match the oracle on the chronological window")


def test_ring_store_in_a_graph():
    """The store and a counter increment captured together; each replay
    writes the next slot, as the oracle does step by step."""
    from oracle import rkv_oracle as O
    spec = syn.config(1).with_(name="ring-graph", seed=62, num_seqs=2, num_layers=2, num_q_heads=4,
                               num_kv_heads=1, window=4, budget=64, buffer=16, lens=(80, 80))
    cfg = config_of(spec)
    rng = np.random.default_rng([62])
    q_h = step_queries(spec, rng, spec.num_layers)
    q = to_dev(q_h)
    ring = torch.zeros((spec.num_layers, spec.num_seqs, spec.num_q_heads, spec.window, spec.head_dim),
                       dtype=torch.int16, device="cuda")
    steps = torch.tensor([3, 10], dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        B.rkv_window_store(cfg, 0, spec.num_layers, q, spec.num_seqs, steps, ring,
                           torch.cuda.current_stream())
        steps.add_(1)
    torch.cuda.synchronize()
    want = np.zeros(tuple(ring.shape), dtype=np.uint16)
    st = np.array([3, 10], dtype=np.int64)
    for rep in range(6):
        ring.view(-1)[:1].add_(0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = O.window_store(want, q_h, 0, st + rep, spec.window)
        assert np.array_equal(to_host(ring, "bf16"), want), f"replay {rep}"
    assert torch.equal(steps.cpu(), torch.tensor([9, 16], dtype=torch.int32))
    log("ring store: 6 graph replays write the slots of steps 3.. and 10..")
