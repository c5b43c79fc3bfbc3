"""Caches whose layers sit apart in one allocation (rkv_cache.layer_stride):
padding between the layers holds a canary, and every entry point gives the
bytes it gives on the packed layout -- scores, keep rows, compacted rows,
FREE_BLOCKS, the Gram redundancy -- and never writes the padding."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import ContigCase, PagedCase, canary_value, config_of, log
from kv_cache_compression_decode_amd import binding as B
from kv_cache_compression_decode_amd.step import RKVStep


def free_capacity(case, how):
    """FREE_BLOCKS entries: the closed-form count, or for device lengths the
    worst case rkv_step_device requires (every sequence at the longest)."""
    spec = case.spec
    if spec.layout != "paged" or how != "rkv_step_device":
        return case.free_capacity
    bs = spec.block_size
    return spec.num_seqs * max(0, -(-int(case.lens0.max()) // bs) - -(-spec.budget // bs))

pytestmark = pytest.mark.gpu

PAD = 8 * 37          # elements of padding after each layer (a multiple of 16 bytes)

CASES = [
    # fused single pass (N <= 1280, bf16)
    syn.config(1).with_(name="stride-fused", seed=51, num_seqs=2, num_layers=3, lens=(1152, 1200)),
    # key spans (N > 1280) on the three kernels
    syn.config(1).with_(name="stride-long", seed=52, num_seqs=2, num_layers=2, lens=(2000, 1300)),
    # fp32: the two-kernel scoring
    syn.config(0).with_(name="stride-f32", seed=53, num_seqs=2, num_layers=3, lens=(300, 170)),
    # paged, short and long units
    syn.config(3).with_(name="stride-paged", seed=54, num_seqs=2, num_layers=3, budget=512,
                        buffer=64, num_blocks=300, lens=(700, 1500)),
    syn.config(3).with_(name="stride-paged-bs32", seed=55, num_seqs=2, num_layers=2, budget=256,
                        buffer=32, block_size=32, num_blocks=64, lens=(400, 300)),
]


def padded(case):
    """Copies of case.k / case.v with PAD elements of canary after each layer;
    returns (k, v, stride) with k, v of shape (L, stride)."""
    L = case.k.shape[0]
    per = case.k[0].numel()
    stride = per + PAD
    out = []
    for t in (case.k, case.v):
        big = torch.full((L, stride), canary_value(case.spec), dtype=t.dtype, device="cuda")
        big[:, :per] = t.reshape(L, -1)
        out.append(big)
    return out[0], out[1], stride


def make_cache(case, k, v, stride):
    if case.spec.layout == "paged":
        return B.make_cache(k, v, num_blocks=case.spec.num_blocks, block_table=case.bt_dev,
                            max_blocks_per_seq=case.bt.shape[1], layer_stride=stride)
    return B.make_cache(k, v, capacity=case.cap, layer_stride=stride)


def run(case, cache, how):
    spec = case.spec
    step = RKVStep(config_of(spec), spec.num_seqs, int(case.lens0.max()),
                   keep_parts=how == "three_calls", free_capacity=free_capacity(case, how))
    step.scores.fill_(float("nan"))
    step.keep.fill_(-7)
    if step.free_blocks is not None:
        step.free_blocks.fill_(-9)
    lens = case.lens0.astype(np.int32).copy()
    if how == "three_calls":
        step(cache, case.q, lens)
    elif how == "rkv_step":
        step.fused(cache, case.q, lens)
    else:
        d_lens = torch.from_numpy(case.lens0.astype(np.int32)).cuda()
        step.device(cache, case.q, d_lens)
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
@pytest.mark.parametrize("how", ["three_calls", "rkv_step", "rkv_step_device"])
def test_padded_layers_match_packed(spec, how):
    log(f"layer stride: {spec.name} via {how}")
    case = PagedCase(spec) if spec.layout == "paged" else ContigCase(spec)
    L = spec.num_layers
    per = case.k[0].numel()
    k_pad, v_pad, stride = padded(case)
    ref = run(case, case.cache, how)                      # packed, compacted in place
    got = run(case, make_cache(case, k_pad, v_pad, stride), how)
    assert torch.equal(torch.nan_to_num(got.scores, nan=-1.0), torch.nan_to_num(ref.scores, nan=-1.0))
    assert torch.equal(got.keep, ref.keep)
    if ref.free_blocks is not None:
        assert torch.equal(got.free_blocks, ref.free_blocks)
    assert torch.equal(k_pad[:, :per], case.k.reshape(L, -1)), "compacted K differs"
    assert torch.equal(v_pad[:, :per], case.v.reshape(L, -1)), "compacted V differs"
    can = canary_value(spec)
    assert bool((k_pad[:, per:] == can).all()) and bool((v_pad[:, per:] == can).all()), \
        "the padding between layers was written"


@pytest.mark.parametrize("spec", [c for c in CASES if c.dtype == "bf16"], ids=lambda s: s.name)
def test_padded_layers_gram(spec):
    log(f"layer stride, Gram: {spec.name}")
    case = PagedCase(spec) if spec.layout == "paged" else ContigCase(spec)
    k_pad, v_pad, stride = padded(case)
    cfg = config_of(spec)
    maxn = int(case.lens0.max())
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    outs = []
    for cache in (case.cache, make_cache(case, k_pad, v_pad, stride)):
        red = torch.full((rows * maxn,), float("nan"), device="cuda")
        B.rkv_redundancy_gram(cfg, cache, spec.num_seqs, case.lens0.astype(np.int32), red, maxn)
        torch.cuda.synchronize()
        outs.append(torch.nan_to_num(red, nan=-1.0))
    assert torch.equal(outs[0], outs[1])
