"""The seeded input generators: determinism, shapes and the stated recipe."""
import numpy as np
import pytest
import torch

import rkv_synth as syn

pytestmark = pytest.mark.cpu


def test_bf16_encoding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0, 1e-30],
                                 dtype=np.float32)])
    ours = syn.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_chunks_regenerate_identically():
    spec = syn.config(1)
    a = syn.keys(spec, 0, 5)
    b = syn.keys(spec, 0, 5)
    assert np.array_equal(a, b)
    assert a.shape == (8, 1152, 128) and a.dtype == np.uint16
    assert not np.array_equal(a, syn.keys(spec, 0, 6))
    q = syn.queries(spec, 0, 3)
    assert q.shape == (32, 8, 128)


def test_scatter_duplicates_recipe():
    spec = syn.config(1)
    plan = syn.dup_plan(spec, 0, 1152)
    assert len(plan) == int(0.3 * 1152)
    dsts = [d for d, _, _ in plan]
    assert dsts == sorted(dsts) and len(set(dsts)) == len(dsts)
    assert all(0 <= s < d for d, s, _ in plan)
    # a duplicated key is its source plus small noise (before bf16 rounding)
    k = syn._keys_f32(spec, 0, 0, 1152, plan)
    d, s, _ = plan[-1]
    assert np.abs(k[:, d] - k[:, s]).max() < 0.1
    assert np.abs(k[:, d] - k[:, s]).max() > 0


def test_runs_recipe():
    spec = syn.config(4)
    plan = syn.dup_plan(spec, 3, 1152)
    cov = sum(length for _, _, length in plan)
    assert cov >= 0.4 * 1152
    last_end = -1
    for dst, src, length in plan:
        assert 16 <= length <= 64
        assert src + length <= dst
        assert dst > last_end
        last_end = dst + length - 1
    assert last_end < 1152


def test_ragged_lengths_and_fractions():
    spec = syn.config(2)
    lens = syn.seq_lens(spec)
    assert lens.shape == (16,)
    assert lens.min() >= spec.budget + 1 and lens.max() <= spec.budget + 128
    fr = []
    for s in range(16):
        plan = syn.dup_plan(spec, s, int(lens[s]))
        fr.append(len(plan) / int(lens[s]))
    assert 0.09 <= min(fr) and max(fr) <= 0.5


def test_block_table_is_a_permutation_prefix():
    spec = syn.config(3)
    bt = syn.block_table(spec)
    assert bt.shape == (8, 272)
    flat = bt.ravel()
    assert len(np.unique(flat)) == flat.size
    assert flat.min() >= 0 and flat.max() < 65536


def test_key_means_shared_across_sequences():
    spec = syn.config(4)
    mu = syn.key_means(spec, 7)
    assert mu.shape == (8, 128)
    assert 0.3 < mu.std() < 0.7


def test_small_contiguous_build_has_canary_tail():
    spec = syn.config(2).with_(num_seqs=3, num_layers=2, len_range=(2049, 2060))
    k, v = syn.build_contiguous(spec, capacity=2100)
    lens = syn.seq_lens(spec)
    assert k.shape == (2, 3, 4, 2100, 128)
    for s in range(3):
        assert np.all(k[:, s, :, lens[s]:] == syn.CANARY_BF16)
        assert np.array_equal(k[1, s, :, :lens[s]], syn.keys(spec, s, 1))
        assert np.array_equal(v[0, s, :, :lens[s]], syn.values(spec, s, 0))
