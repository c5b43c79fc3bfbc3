"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
same seeded inputs.  Scores within 1e-3 (relative; fp32 accumulation vs
float64), keep sets identical to the oracle's rule applied to the GPU's own
scores and to the float64 oracle outside the threshold band, compacted K/V
and FREE_BLOCKS bit-exact."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import (ContigCase, PagedCase, check_unit, check_units_parallel, config_of,
                         keep_invariants_on_device, log, make_case, one_unit_per_layer, run_step,
                         sample_units, to_host)
from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.gpu


def check_all(case, step, units, tag):
    near = 0
    for (s, l, h) in units:
        near += check_unit(case, step, s, l, h, tag)
    log(f"{tag}: {len(units)} units match the oracle ({near} keep differences inside the band)")


def check_untriggered(case, step, lens_after):
    """Sequences below the trigger: cache, scores and keep rows untouched."""
    spec = case.spec
    thr = spec.budget + spec.buffer
    for s in range(spec.num_seqs):
        n = int(case.lens0[s])
        if n >= thr:
            assert lens_after[s] == spec.budget
            continue
        assert lens_after[s] == n
        for l in range(spec.num_layers):
            for h in range(spec.num_kv_heads):
                row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
                assert torch.isnan(step.scores[row * step.max_len:(row + 1) * step.max_len]).all()
                assert (step.keep[row * spec.budget:(row + 1) * spec.budget] == -7).all()
        if isinstance(case, ContigCase):
            k = to_host(case.k[:, s], spec.dtype)
            v = to_host(case.v[:, s], spec.dtype)
            assert np.array_equal(k, case.k_host[:, s]) and np.array_equal(v, case.v_host[:, s])


def check_tail_untouched(case):
    """Contiguous: slots >= budget of triggered units keep their old rows."""
    spec = case.spec
    for s in range(spec.num_seqs):
        if case.lens0[s] < spec.budget + spec.buffer:
            continue
        k = to_host(case.k[:, s, :, spec.budget:], spec.dtype)
        assert np.array_equal(k, case.k_host[:, s, :, spec.budget:])


# ------------------------------------------------------------------ workloads

def test_config0_tiny_f32():
    spec = syn.config(0)
    case = ContigCase(spec)
    step, lens = run_step(case)
    check_all(case, step, sample_units(spec, 10**9), "tiny-f32")
    check_tail_untouched(case)
    assert lens[0] == spec.budget


def test_config1_llama8b_full():
    spec = syn.config(1)
    case = ContigCase(spec)
    step, lens = run_step(case)
    check_all(case, step, sample_units(spec, 10**9), "llama8b-1seq")
    check_tail_untouched(case)


SMALL = {
    # several 256-key chunks, a ragged tail, one sequence below the trigger
    "ragged-bf16-d128": syn.config(1).with_(name="ragged", seed=11, num_seqs=3, num_layers=2,
                                             num_q_heads=8, num_kv_heads=2, budget=256, buffer=32,
                                             lens=(777, 250, 300)),
    "bf16-d64-mha": syn.config(1).with_(name="d64", seed=12, num_seqs=2, num_layers=2,
                                         num_q_heads=4, num_kv_heads=4, head_dim=64, window=4,
                                         budget=200, buffer=40, lens=(513, 240)),
    "wide-group-rt9": syn.config(1).with_(name="rt9", seed=13, num_seqs=1, num_layers=1,
                                           num_q_heads=64, num_kv_heads=8, window=16, budget=300,
                                           buffer=20, lens=(600,)),
    "gqa7-rt4": syn.config(2).with_(name="g7", seed=14, num_seqs=2, num_layers=2, budget=400,
                                     buffer=64, len_range=None, lens=(464, 1000)),
    "lambda0": syn.config(1).with_(name="l0", seed=15, num_seqs=1, num_layers=2, mix_lambda=0.0,
                                    budget=256, buffer=64, lens=(400,)),
    "lambda1": syn.config(1).with_(name="l1", seed=16, num_seqs=1, num_layers=2, mix_lambda=1.0,
                                    budget=256, buffer=64, lens=(400,)),
    "window1-keep1": syn.config(1).with_(name="w1", seed=17, num_seqs=1, num_layers=1,
                                          num_q_heads=8, num_kv_heads=8, window=1, budget=2,
                                          buffer=50, lens=(70,)),
    "at-trigger-and-capacity": syn.config(1).with_(name="edge", seed=18, num_seqs=2, num_layers=1,
                                                   budget=128, buffer=16, lens=(144, 2049)),
    "f32-d128": syn.config(0).with_(name="f32d128", seed=19, num_seqs=2, num_layers=2,
                                    num_q_heads=8, num_kv_heads=2, head_dim=128, budget=200,
                                    buffer=30, lens=(300, 529)),
    "paged-bs16-partial": syn.config(3).with_(name="p16", seed=20, num_seqs=3, num_layers=2,
                                              num_q_heads=8, num_kv_heads=2, budget=300,
                                              buffer=45, num_blocks=300, lens=(345, 500, 200)),
    "paged-bs32": syn.config(3).with_(name="p32", seed=21, num_seqs=2, num_layers=2,
                                      num_q_heads=8, num_kv_heads=2, budget=250, block_size=32,
                                      buffer=40, num_blocks=100, lens=(290, 700)),
    "runs-dups": syn.config(4).with_(name="runs", seed=22, num_seqs=2, num_layers=2,
                                     lens=(1152, 1152)),
    # the largest window-row count the kernels accept: 71 query heads on one kv head, w = 2
    "window-rows-142": syn.config(1).with_(name="gw142", seed=23, num_seqs=1, num_layers=1,
                                           num_q_heads=71, num_kv_heads=1, window=2, budget=200,
                                           buffer=40, lens=(400,)),
    # paged block sizes at both ends of the supported range
    "paged-bs1": syn.config(3).with_(name="p1", seed=24, num_seqs=2, num_layers=2, num_q_heads=8,
                                     num_kv_heads=2, budget=60, buffer=10, block_size=1,
                                     num_blocks=200, lens=(70, 90)),
    "paged-bs1024-d64": syn.config(3).with_(name="p1024", seed=25, num_seqs=2, num_layers=2,
                                            num_q_heads=4, num_kv_heads=2, head_dim=64,
                                            budget=1500, buffer=100, block_size=1024,
                                            num_blocks=8, lens=(1600, 2100)),
    # units longer than one workgroup holds are scored as key spans on several
    # workgroups: 11 spans for the 12801-token sequence, so the 10-token one
    # in the same launch has spans without any key
    "spans-empty": syn.config(1).with_(name="spe", seed=26, num_seqs=2, num_layers=1,
                                       num_q_heads=4, num_kv_heads=1, budget=9, buffer=1,
                                       lens=(10, 12801)),
    "spans-d64": syn.config(1).with_(name="spd", seed=27, num_seqs=1, num_layers=2, num_q_heads=4,
                                     num_kv_heads=2, head_dim=64, budget=2000, buffer=100,
                                     lens=(3100,)),
    # key spans over a paged cache at head_dim 64 (units above 2560 keys)
    "spans-paged-d64": syn.config(3).with_(name="spp", seed=28, num_seqs=2, num_layers=2,
                                           num_q_heads=4, num_kv_heads=2, head_dim=64, budget=2600,
                                           buffer=100, num_blocks=500, lens=(2750, 3300)),
    # fp32 caches in the paged layout
    "f32-paged": syn.config(3).with_(name="f32p", seed=29, dtype="f32", num_seqs=2, num_layers=2,
                                     num_q_heads=8, num_kv_heads=2, budget=300, buffer=40,
                                     num_blocks=100, lens=(345, 500)),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small(name):
    spec = SMALL[name]
    kw = {}
    if spec.layout != "paged" and name != "at-trigger-and-capacity":
        kw["capacity"] = int(syn.seq_lens(spec).max()) + 5
    case = make_case(spec, **kw)
    step, lens = run_step(case)
    check_all(case, step, sample_units(spec, 10**9), name)
    check_untriggered(case, step, lens)
    if spec.layout == "paged":
        check_free_blocks(case, step)
    else:
        check_tail_untouched(case)


def check_free_blocks(case, step):
    from oracle import rkv_oracle as O
    spec = case.spec
    expect, counts = [], []
    for s in range(spec.num_seqs):
        n = int(case.lens0[s])
        if O.is_triggered(n, spec.budget, spec.buffer):
            ids = O.free_blocks(case.bt[s], n, spec.budget, spec.block_size)
        else:
            ids = []
        expect += ids
        counts.append(len(ids))
    assert list(step.free_counts) == counts
    got = step.free_blocks[:len(expect)].cpu().numpy().tolist() if expect else []
    assert got == expect


@pytest.mark.timeout(600)
def test_config2_ragged_literal():
    """Lengths uniform in [B+1, B+128]: only N = B+128 triggers; the rest
    pass through untouched in the same launch."""
    spec = syn.config(2)
    case = ContigCase(spec)
    step, lens = run_step(case)
    trig = [s for s in range(spec.num_seqs) if case.lens0[s] >= spec.budget + spec.buffer]
    log(f"config 2 at seed {spec.seed}: lengths {case.lens0.tolist()}, triggered {trig}")
    check_untriggered(case, step, lens)
    # every unit of the triggered sequence (28 layers x 4 kv heads)
    check_units_parallel(case, step, sample_units(spec, 10**9), "qwen7b-ragged16")


@pytest.mark.timeout(600)
def test_config2_all_triggered_diagnostic():
    """Diagnostic, not one of the five workloads: config 2 with buffer 1, so
    all 16 sequences trigger at their ragged lengths in one launch."""
    spec = syn.config(2).with_(buffer=1)
    case = ContigCase(spec)
    step, lens = run_step(case)
    assert (lens == spec.budget).all()
    # one unit per (sequence, layer): 448 units
    check_units_parallel(case, step, one_unit_per_layer(spec, seed=2), "ragged-all-trigger")
    assert keep_invariants_on_device(step, spec, case.lens0) == 16 * 28 * 4
    check_tail_untouched(case)


@pytest.mark.timeout(900)
def test_config3_paged_full():
    spec = syn.config(3)
    log("config 3: building 128 GiB of pools")
    case = PagedCase(spec)
    ref_blocks = torch.from_numpy(np.unique(case.bt).astype(np.int64)).to(case.k.device)
    pristine_k = case.k.index_select(1, ref_blocks)
    pristine_v = case.v.index_select(1, ref_blocks)
    log("config 3: running the step")
    step, lens = run_step(case)
    check_free_blocks(case, step)
    assert len(step.free_counts) == 8 and all(c == 16 for c in step.free_counts)
    assert keep_invariants_on_device(step, spec, case.lens0) == 2048
    # one unit per (sequence, layer) against the oracle: 256 units
    check_units_parallel(case, step, one_unit_per_layer(spec, seed=3), "llama8b-paged8")
    # every unit's compacted rows against a gather of the pristine blocks
    pos = {int(b): i for i, b in enumerate(ref_blocks.tolist())}
    keep = step.keep.view(spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.budget).long()
    bs, nkeep = spec.block_size, spec.budget // spec.block_size
    for s in range(spec.num_seqs):
        nb = -(-int(case.lens0[s]) // bs)
        src = torch.tensor([pos[int(b)] for b in case.bt[s, :nb]], device=case.k.device)
        dst = torch.from_numpy(case.bt[s, :nkeep].astype(np.int64)).to(case.k.device)
        for pool, pristine in ((case.k, pristine_k), (case.v, pristine_v)):
            for l in range(spec.num_layers):
                # logical rows of every kv head: (H, nb * bs, d)
                old = pristine[l].index_select(0, src).permute(1, 0, 2, 3).reshape(spec.num_kv_heads, nb * bs, -1)
                want = torch.gather(old, 1, keep[l, s].unsqueeze(-1).expand(-1, -1, old.shape[-1]))
                got = pool[l].index_select(0, dst).permute(1, 0, 2, 3).reshape(spec.num_kv_heads, nkeep * bs, -1)
                assert torch.equal(got, want), (s, l)
    log("config 3: all 2048 units compacted as their keep lists say")
    del pristine_k, pristine_v
    # blocks nobody references still hold the canary
    ref = np.zeros(spec.num_blocks, dtype=bool)
    ref[case.bt.ravel()] = True
    unref = torch.from_numpy(~ref).to(case.k.device)
    from gpu_harness import canary_value
    cv = canary_value(spec)
    for l in range(spec.num_layers):
        assert bool((case.k[l][unref] == cv).all()) and bool((case.v[l][unref] == cv).all()), l
    log("config 3: unreferenced blocks untouched")


@pytest.mark.timeout(900)
def test_config4_70b_full():
    spec = syn.config(4)
    log("config 4: generating 12 GB of K/V")
    case = ContigCase(spec, keep_host=True)
    k0 = case.k.clone()
    v0 = case.v.clone()
    log("config 4: running the step")
    step, lens = run_step(case, keep_parts=False)
    assert keep_invariants_on_device(step, spec, case.lens0) == 20480
    # one unit per (sequence, layer) against the oracle: 2560 units
    check_units_parallel(case, step, one_unit_per_layer(spec, seed=4), "70b-batch32")
    # property at full size: every compacted row is the original row keep[i]
    keep = step.keep.view(spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.budget).long()
    for l in range(spec.num_layers):
        idx = keep[l].unsqueeze(-1).expand(-1, -1, -1, spec.head_dim)
        assert torch.equal(case.k[l, :, :, :spec.budget], torch.gather(k0[l], 2, idx)), l
        assert torch.equal(case.v[l, :, :, :spec.budget], torch.gather(v0[l], 2, idx)), l
    log("config 4: all 20480 units compacted as their keep lists say")


# ------------------------------------------------------------------ properties

def test_deterministic_bitwise():
    spec = syn.config(1).with_(num_layers=4)
    outs = []
    for _ in range(2):
        case = ContigCase(spec)
        step, _ = run_step(case)
        outs.append((step.scores.clone(), step.keep.clone(), case.k.clone(), case.v.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
@pytest.mark.parametrize("pattern", ["shift1", "max-shift", "none", "random", "blocks"])
def test_adversarial_compaction(layout, pattern):
    """In-place compaction for keep lists the selection would rarely produce,
    against numpy fancy indexing (the oracle's gather)."""
    from oracle import rkv_oracle as O
    base = syn.config(3) if layout == "paged" else syn.config(1)
    spec = base.with_(name="adv", seed=30, num_seqs=2, num_layers=2, num_q_heads=8,
                      num_kv_heads=2, budget=700, buffer=50, lens=(1100, 900), num_blocks=200)
    case = make_case(spec)
    n_of = [int(x) for x in case.lens0]
    rng = np.random.default_rng(5)
    keep = np.empty((spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.budget), np.int32)
    for l in range(spec.num_layers):
        for s in range(spec.num_seqs):
            for h in range(spec.num_kv_heads):
                n, b = n_of[s], spec.budget
                if pattern == "shift1":
                    row = np.arange(1, b + 1)
                elif pattern == "max-shift":
                    row = np.arange(n - b, n)
                elif pattern == "none":
                    row = np.arange(b)
                elif pattern == "blocks":
                    row = np.sort(np.concatenate([np.arange(0, 100), np.arange(n - (b - 100), n)]))
                else:
                    row = np.sort(rng.choice(n, size=b, replace=False))
                keep[l, s, h] = row
    before = {(s, l, h): case.unit_rows(s, l, h) for s in range(spec.num_seqs)
              for l in range(spec.num_layers) for h in range(spec.num_kv_heads)}
    keep_dev = torch.from_numpy(keep).cuda()
    lens = case.lens0.astype(np.int32).copy()
    fb = torch.zeros(max(1, case.free_capacity), dtype=torch.int32, device="cuda")
    counts = np.zeros(spec.num_seqs, np.int32)
    B.rkv_compact(config_of(spec), case.cache, spec.num_seqs, lens, keep_dev, fb,
                  case.free_capacity, counts)
    torch.cuda.synchronize()
    for (s, l, h), (kr, vr) in before.items():
        gk, gv = case.gpu_rows(s, l, h, spec.budget)
        assert np.array_equal(gk, O.compact_rows(kr, keep[l, s, h])), (pattern, s, l, h)
        assert np.array_equal(gv, O.compact_rows(vr, keep[l, s, h])), (pattern, s, l, h)


def test_exact_ties_keep_lower_position():
    """Exact duplicate keys give bit-identical scores on the GPU; with lam = 0
    the later copy of each duplicated pair is evicted first."""
    from oracle import rkv_oracle as O
    spec = syn.config(1).with_(name="ties", seed=40, num_seqs=1, num_layers=1, num_q_heads=4,
                               num_kv_heads=1, budget=100, buffer=20, lens=(120,),
                               mix_lambda=0.0, dup_frac=0.0)
    case = ContigCase(spec)
    k = case.k_host.copy()
    # tokens 50..69 become exact copies of 10..29
    k[0, 0, 0, 50:70] = k[0, 0, 0, 10:30]
    case.k_host = k
    case.k = torch.from_numpy(k.view(np.int16)).cuda()
    case.cache = B.make_cache(case.k, case.v, capacity=case.cap)
    step, _ = run_step(case)
    g = step.scores[:120].cpu().numpy()
    assert np.array_equal(g[10:30], g[50:70]), "duplicate keys must score identically"
    check_unit(case, step, 0, 0, 0, "ties")
    keep = step.keep[:spec.budget].cpu().numpy()
    assert np.array_equal(keep, O.select_keep(g.astype(np.float64), 120, 100, 8))


def test_zero_norm_keys():
    """A zero key has redundancy 0 and contributes nothing to the others."""
    spec = syn.config(1).with_(name="zero", seed=41, num_seqs=1, num_layers=1, num_q_heads=8,
                               num_kv_heads=2, budget=100, buffer=28, lens=(128,))
    case = ContigCase(spec)
    k = case.k_host.copy()
    k[0, 0, :, [3, 77]] = 0
    case.k_host = k
    case.k = torch.from_numpy(k.view(np.int16)).cuda()
    case.cache = B.make_cache(case.k, case.v, capacity=case.cap)
    step, _ = run_step(case)
    red = step.redundancy[:128].cpu().numpy()
    assert red[3] == 0.0 and red[77] == 0.0
    for h in range(2):
        check_unit(case, step, 0, 0, h, "zero-keys")
