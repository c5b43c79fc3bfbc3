"""Head-shared selection (one keep set per sequence and layer, ranked by the
float32 sum of the KV heads' scores) through the C ABI, against the oracle,
and rkv_step against the three calls in that mode."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import (ContigCase, check_layer_shared, config_of, log, make_case, run_step,
                         to_host)
from kv_cache_compression_decode_amd.step import RKVStep

pytestmark = pytest.mark.gpu

CASES = {
    "llama8b-1seq": syn.config(1),
    "ragged-bf16": syn.config(1).with_(name="sh-r", seed=71, num_seqs=3, num_layers=2,
                                       num_q_heads=8, num_kv_heads=2, budget=256, buffer=32,
                                       lens=(777, 250, 300)),
    "paged-bs16": syn.config(3).with_(name="sh-p", seed=72, num_seqs=3, num_layers=2,
                                      num_q_heads=8, num_kv_heads=4, budget=300, buffer=45,
                                      num_blocks=400, lens=(345, 1280, 200)),
    "long-2176": syn.config(2).with_(num_seqs=2, num_layers=2, len_range=None, lens=(2176, 2100)),
    "d64-mha": syn.config(1).with_(name="sh-d64", seed=73, num_seqs=2, num_layers=2, num_q_heads=4,
                                   num_kv_heads=4, head_dim=64, window=4, budget=500, buffer=40,
                                   lens=(700, 540)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_shared_against_oracle(name):
    spec = CASES[name]
    case = make_case(spec)
    step, lens = run_step(case, shared=True)
    thr = spec.budget + spec.buffer
    near = 0
    for s in range(spec.num_seqs):
        n = int(case.lens0[s])
        if n < thr:
            assert lens[s] == n
            continue
        assert lens[s] == spec.budget
        for l in range(spec.num_layers):
            near += check_layer_shared(case, step, s, l, name)
    log(f"{name}: head-shared selection matches the oracle ({near} keep differences in the band)")


def test_shared_single_head_equals_per_head():
    """One KV head: the shared rule is the per-head rule, bit for bit."""
    spec = syn.config(0)
    outs = []
    for shared in (False, True):
        case = ContigCase(spec)
        step, lens = run_step(case, shared=shared)
        outs.append((step.keep.clone(), step.scores.clone(), case.k.clone(), case.v.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["llama8b-1seq", "paged-bs16"])
def test_shared_step_equals_three_calls(name):
    spec = CASES[name]
    res = []
    for fused in (False, True):
        case = make_case(spec)
        cfg = config_of(spec, shared=True)
        st = RKVStep(cfg, spec.num_seqs, int(case.lens0.max()), free_capacity=case.free_capacity)
        st.keep.fill_(-7)
        lens = case.lens0.astype(np.int32).copy()
        (st.fused if fused else st)(case.cache, case.q, lens, torch.cuda.current_stream())
        torch.cuda.synchronize()
        fb = None if st.free_blocks is None else st.free_blocks.clone()
        res.append((st.keep.clone(), case.k.clone(), case.v.clone(), lens.copy(),
                    st.free_counts.copy(), fb))
    (k0, K0, V0, l0, c0, f0), (k1, K1, V1, l1, c1, f1) = res
    assert torch.equal(k0, k1) and torch.equal(K0, K1) and torch.equal(V0, V1)
    assert np.array_equal(l0, l1) and np.array_equal(c0, c1)
    if f0 is not None:
        assert torch.equal(f0, f1)
    log(f"{name}: rkv_step with head-shared selection equals the three calls")
