"""Device checks and the workspace's status word: a key-span wait that gives
up, and block-table ids outside the pool (cfg.check_block_table).  Every
kernel exits normally; the status is reported; the cache, the keep rows and
FREE_BLOCKS keep their input contents.  The failures are forced from the
host: a zero wait bound (rkv_set_span_wait_us) and a block id planted in the
table that points past the declared pool but inside the allocation, so that
even a kernel that missed the check would only read allocated memory."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import (ContigCase, PagedCase, canary_value, check_unit, config_of, log,
                         run_step, sample_units)
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

# bf16 units longer than 1280 keys (head_dim 128) take the key-span launches
LONG = syn.config(1).with_(name="status-long", seed=41, num_seqs=3, num_layers=2, budget=1024,
                           buffer=128, lens=(2100, 1500, 900))


def snapshot(case):
    return case.k.clone(), case.v.clone()


def same_cache(case, snap):
    return torch.equal(case.k, snap[0]) and torch.equal(case.v, snap[1])


@pytest.mark.parametrize("entry", ["three_calls", "rkv_step", "rkv_step_device"])
def test_span_timeout_leaves_cache(entry):
    log(f"span timeout via {entry}")
    case = ContigCase(LONG)
    cfg = config_of(LONG)
    maxn = int(case.lens0.max())
    step = RKVStep(cfg, LONG.num_seqs, maxn, free_capacity=0)
    step.keep.fill_(-7)
    snap = snapshot(case)
    lens = case.lens0.astype(np.int32).copy()
    prev = B.rkv_set_span_wait_us(0)
    try:
        if entry == "three_calls":
            step(case.cache, case.q, lens)
            flags = step.status()
        elif entry == "rkv_step":
            step.fused(case.cache, case.q, lens)
            flags = step.status()
        else:
            d_lens = torch.from_numpy(case.lens0.astype(np.int32)).cuda()
            step.device(case.cache, case.q, d_lens)
            flags = step.device_status()
        torch.cuda.synchronize()
    finally:
        B.rkv_set_span_wait_us(prev)
    assert flags == B.RKV_DEVICE_SPAN_TIMEOUT, flags
    assert same_cache(case, snap), "the cache changed after a failed device check"
    assert bool((step.keep == -7).all()), "keep rows were written after a failed device check"
    with pytest.raises(B.RkvError) as e:
        B._check(B.load().rkv_device_status(B._ptr(step.workspace if entry != "rkv_step_device"
                                                     else step.dev_ws), None, None))
    assert e.value.status == B.RKV_ERR_DEVICE_CHECK
    # the same workspace, the default bound: the step runs and the word is clear
    lens = case.lens0.astype(np.int32).copy()
    step(case.cache, case.q, lens)
    assert step.status() == 0
    torch.cuda.synchronize()
    for s, l, h in sample_units(LONG, 6, seed=3):
        check_unit(case, step, s, l, h, "after a timeout")


def _paged_with_slack(spec, slack):
    """The case's pools copied into pools of num_blocks + slack blocks per
    layer (the extra blocks hold the canary); the cache declares num_blocks,
    so its layer stride is that of the larger pool."""
    case = PagedCase(spec)
    L, nb, hk, bs, d = case.k.shape
    per = hk * bs * d
    big_k = torch.full((L, (nb + slack) * per), canary_value(spec), dtype=case.k.dtype,
                       device="cuda")
    big_v = big_k.clone()
    big_k[:, :nb * per] = case.k.reshape(L, -1)
    big_v[:, :nb * per] = case.v.reshape(L, -1)
    case.k = big_k[:, :nb * per].view(L, nb, hk, bs, d)   # views for gpu_rows
    case.v = big_v[:, :nb * per].view(L, nb, hk, bs, d)
    case.big_k, case.big_v = big_k, big_v
    case.stride = (nb + slack) * per
    case.cache = B.make_cache(big_k, big_v, num_blocks=nb, block_table=case.bt_dev,
                              max_blocks_per_seq=case.bt.shape[1], layer_stride=case.stride)
    return case


PAGED_SHORT = syn.config(3).with_(name="status-paged", seed=42, num_seqs=2, num_layers=2,
                                  budget=512, buffer=64, num_blocks=256, lens=(700, 576))
PAGED_LONG = PAGED_SHORT.with_(name="status-paged-long", seed=43, budget=1024, buffer=128,
                               lens=(1900, 1200))


@pytest.mark.parametrize("spec", [PAGED_SHORT, PAGED_LONG], ids=lambda s: s.name)
@pytest.mark.parametrize("entry", ["three_calls", "rkv_step", "rkv_step_device"])
def test_bad_block_id(spec, entry):
    log(f"bad block id: {spec.name} via {entry}")
    case = _paged_with_slack(spec, slack=8)
    nb = spec.num_blocks
    cfg = B.make_config(spec.num_layers, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                        spec.budget, spec.buffer, spec.window, spec.mix_lambda, spec.dtype,
                        "paged", spec.block_size, check_block_table=True)
    maxn = int(case.lens0.max())

    def run(c):
        step = RKVStep(c, spec.num_seqs, maxn, free_capacity=free_capacity(case, entry))
        step.keep.fill_(-7)
        if step.free_blocks is not None:
            step.free_blocks.fill_(-9)
        lens = case.lens0.astype(np.int32).copy()
        if entry == "three_calls":
            step(case.cache, case.q, lens)
            flags = step.status()
        elif entry == "rkv_step":
            step.fused(case.cache, case.q, lens)
            flags = step.status()
        else:
            d_lens = torch.from_numpy(case.lens0.astype(np.int32)).cuda()
            step.device(case.cache, case.q, d_lens)
            flags = step.device_status()
        torch.cuda.synchronize()
        return step, flags

    # a valid table with the check on: no flag, and the results of the check off
    snap = (case.big_k.clone(), case.big_v.clone())
    step_on, flags = run(cfg)
    assert flags == 0
    res_on = (step_on.keep.clone(), case.big_k.clone(), case.big_v.clone())
    case.big_k.copy_(snap[0])
    case.big_v.copy_(snap[1])
    cfg_off = config_of(spec)
    step_off, flags = run(cfg_off)
    assert flags == 0
    assert torch.equal(step_off.keep, res_on[0])
    assert torch.equal(case.big_k, res_on[1]) and torch.equal(case.big_v, res_on[2])
    for s, l, h in sample_units(spec, 4, seed=5):
        check_unit(case, step_off, s, l, h, "check on, valid table")
    case.big_k.copy_(snap[0])
    case.big_v.copy_(snap[1])

    # one id past the declared pool (inside the allocation's slack)
    bad = case.bt.copy()
    bad[spec.num_seqs - 1, 3] = nb + 5
    case.bt_dev.copy_(torch.from_numpy(bad))
    step, flags = run(cfg)
    assert flags == B.RKV_DEVICE_BAD_BLOCK_ID, flags
    assert torch.equal(case.big_k, snap[0]) and torch.equal(case.big_v, snap[1]), \
        "the pool changed after a failed block check"
    assert bool((step.keep == -7).all())
    if step.free_blocks is not None:
        assert bool((step.free_blocks == -9).all())
    case.bt_dev.copy_(torch.from_numpy(case.bt))


def test_status_clear_after_ordinary_steps():
    """Every path clears the word: fused, three calls, device lengths."""
    spec = syn.config(1).with_(name="status-fused", seed=44, num_seqs=2, num_layers=2,
                               lens=(1152, 1200))
    case = ContigCase(spec)
    step, _ = run_step(case, fused=True)
    assert step.status() == 0
    ws = step.workspace
    # plant a flag: the next fused step clears it
    ws[:4] = torch.tensor([3, 0, 0, 0], dtype=torch.uint8, device="cuda")
    lens = case.lens0.astype(np.int32).copy()
    case2 = ContigCase(spec)
    step.fused(case2.cache, case2.q, lens)
    assert step.status() == 0
    ws[:4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    lens = case.lens0.astype(np.int32).copy()
    case3 = ContigCase(spec)
    step(case3.cache, case3.q, lens)
    assert step.status() == 0
    for s, l, h in sample_units(spec, 4, seed=6):
        check_unit(case3, step, s, l, h, "after a planted flag")
