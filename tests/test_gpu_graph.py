"""The step captured in a HIP graph (as the benchmark runs it): every replay,
with eager work and synchronisation between replays, must equal the eager
step bit for bit."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import ContigCase, PagedCase, config_of, log
from kv_cache_compression_decode_amd import binding as B
from kv_cache_compression_decode_amd.step import RKVStep

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("which", ["llama8b-1seq", "paged-small", "spans"])
def test_graph_replays_match_eager(which):
    if which == "llama8b-1seq":
        spec = syn.config(1)
        case = ContigCase(spec)
    elif which == "spans":   # units longer than one workgroup: key-span launches + counter reset
        spec = syn.config(1).with_(name="gspan", seed=51, num_seqs=2, num_layers=2, num_q_heads=4,
                                   num_kv_heads=2, head_dim=64, budget=2000, buffer=100,
                                   lens=(3100, 1500))
        case = ContigCase(spec)
    else:
        spec = syn.config(3).with_(name="pg", seed=50, num_seqs=3, num_layers=2, budget=500,
                                   buffer=60, num_blocks=400, lens=(560, 900, 300))
        case = PagedCase(spec)
    k0, v0 = case.k.clone(), case.v.clone()
    cfg = config_of(spec)
    maxn = int(case.lens0.max())

    def fresh_cache():
        case.k.copy_(k0)
        case.v.copy_(v0)
        torch.cuda.synchronize()

    def sentinel(st):
        # rows of untriggered units are never written: give both runs the same bytes
        st.scores.fill_(-3.0)
        st.keep.fill_(-5)
        if st.free_blocks is not None:
            st.free_blocks.fill_(-9)

    # eager reference
    ref = RKVStep(cfg, spec.num_seqs, maxn, free_capacity=case.free_capacity)
    sentinel(ref)
    lens = case.lens0.astype(np.int32).copy()
    ref(case.cache, case.q, lens, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = (ref.scores.clone(), ref.keep.clone(), case.k.clone(), case.v.clone(),
            None if ref.free_blocks is None else ref.free_blocks.clone())

    fresh_cache()
    step = RKVStep(cfg, spec.num_seqs, maxn, free_capacity=case.free_capacity)
    g = torch.cuda.CUDAGraph()
    lens = case.lens0.astype(np.int32).copy()
    with torch.cuda.graph(g):
        step(case.cache, case.q, lens, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        fresh_cache()
        sentinel(step)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (step.scores, step.keep, case.k, case.v, step.free_blocks)
        for a, b in zip(want, got):
            if a is None:
                continue
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
    log(f"{which}: 3 graph replays equal the eager step")
