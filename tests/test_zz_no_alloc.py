"""rkv_step_noalloc, the entry point that allocates nothing: through the C
ABI it gives rkv_step's bytes (scores, keep rows, compacted cache,
FREE_BLOCKS, lengths), on two calls in a row that share its scratch, the
second with a smaller input; launches that need the scratch (key spans) and
fused ones; a step too large for the scratch is refused."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import PagedCase, ContigCase, check_unit, config_of, log, sample_units
from kv_cache_compression_decode_amd import binding as B
from kv_cache_compression_decode_amd.step import RKVStep

pytestmark = pytest.mark.gpu


def both(case):
    """rkv_step on the case, then rkv_step_noalloc on a fresh copy of it."""
    spec = case.spec
    k0, v0 = case.k.clone(), case.v.clone()
    maxn = int(case.lens0.max())
    ref = RKVStep(config_of(spec), spec.num_seqs, maxn, free_capacity=case.free_capacity)
    ref.scores.fill_(float("nan"))
    ref.keep.fill_(-7)
    lens_ref = case.lens0.astype(np.int32).copy()
    ref.fused(case.cache, case.q, lens_ref)
    torch.cuda.synchronize()
    out = {"k": case.k.clone(), "v": case.v.clone()}
    case.k.copy_(k0)
    case.v.copy_(v0)
    scores = torch.full_like(ref.scores, float("nan"))
    keep = torch.full_like(ref.keep, -7)
    fb = torch.full((max(1, case.free_capacity),), -9, dtype=torch.int32, device="cuda")
    if ref.free_blocks is not None:
        ref_fb = ref.free_blocks[:case.free_capacity].clone()
    counts = np.zeros(spec.num_seqs, np.int32)
    lens = case.lens0.astype(np.int32).copy()
    B.rkv_step_noalloc(config_of(spec), case.cache, case.q, spec.num_seqs, lens, scores, maxn,
                       keep, fb if case.free_capacity else None, case.free_capacity, counts)
    torch.cuda.synchronize()
    assert B.rkv_device_status(None) == 0
    assert np.array_equal(lens, lens_ref)
    assert np.array_equal(counts, ref.free_counts)
    assert torch.equal(torch.nan_to_num(scores, nan=-1.0), torch.nan_to_num(ref.scores, nan=-1.0))
    assert torch.equal(keep, ref.keep)
    assert torch.equal(case.k, out["k"]) and torch.equal(case.v, out["v"])
    if case.free_capacity:
        assert torch.equal(fb[:case.free_capacity], ref_fb)
    return ref


BIG = syn.config(1).with_(name="noalloc-big", seed=61, num_seqs=3, num_layers=3,
                          lens=(2600, 2000, 1300))
SMALL = syn.config(1).with_(name="noalloc-small", seed=62, num_seqs=1, num_layers=2, lens=(1500,))
FUSED = syn.config(1).with_(name="noalloc-fused", seed=63, num_seqs=2, num_layers=2,
                            lens=(1152, 1000))
PAGED = syn.config(3).with_(name="noalloc-paged", seed=64, num_seqs=2, num_layers=2, budget=1024,
                            buffer=128, num_blocks=400, lens=(2500, 1152))


def test_two_calls_second_smaller():
    for spec in (BIG, SMALL):
        log(f"noalloc: {spec.name}")
        case = ContigCase(spec)
        step = both(case)
        for s, l, h in sample_units(spec, 4, seed=1):
            check_unit(case, step, s, l, h, spec.name)


def test_fused_and_paged():
    for spec in (FUSED, PAGED, SMALL):
        log(f"noalloc: {spec.name}")
        case = PagedCase(spec) if spec.layout == "paged" else ContigCase(spec)
        both(case)


def test_too_large_for_the_scratch():
    # 40 sequences of 8192 keys at 32 layers: 40*32*8*32 records of 768 bytes
    spec = syn.config(1).with_(name="noalloc-huge", num_seqs=40, lens=(8192,) * 40)
    cfg = config_of(spec)
    lens = np.array(spec.lens, np.int32)
    cache = B.make_cache(1 << 20, 1 << 20, capacity=8192)   # never read: refused on the host
    with pytest.raises(B.RkvError) as e:
        B.rkv_step_noalloc(cfg, cache, 1 << 20, spec.num_seqs, lens, 1 << 20, 8192, 1 << 20)
    assert e.value.status == B.RKV_ERR_WORKSPACE
    assert list(lens) == [8192] * 40
