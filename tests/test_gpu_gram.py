"""GPU parity of rkv_redundancy_gram (the redundancy signal through the
explicit cosine Gram matrix on the matrix cores) against the CPU oracle's
redundancy, on the same seeded inputs, through the C ABI.

The products take the cached bf16 keys exactly and sum in float32, so the
bar is tighter than the scoring kernels': |R_gpu - R| <= 1e-4 * max|R| + 1e-6
per unit.  Also: agreement with rkv_score's redundancy output (the rank-one
form) within the scoring tolerance, untouched rows and columns, zero keys,
and ragged, paged, head_dim 64 and maximum-length units, in both workgroup
forms (256 and 384 rows; a launch takes the one whose last row block wastes
fewer rows)."""
import numpy as np
import pytest
import torch

import rkv_synth as syn
from gpu_harness import TOL, ContigCase, config_of, log, make_case, sample_units
from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.gpu

GRAM_REL, GRAM_ABS = 1e-4, 1e-6


def run_gram(case, stride=None):
    spec = case.spec
    cfg = config_of(spec)
    maxn = int(case.lens0.max())
    stride = maxn + 3 if stride is None else stride
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    red = torch.full((rows, stride), float("nan"), dtype=torch.float32, device="cuda")
    lens = case.lens0.astype(np.int32).copy()
    B.rkv_redundancy_gram(cfg, case.cache, spec.num_seqs, lens, red, stride)
    torch.cuda.synchronize()
    assert np.array_equal(lens, case.lens0), "lengths changed"
    return red


def row_of(spec, s, l, h):
    return (l * spec.num_seqs + s) * spec.num_kv_heads + h


def check_gram_unit(case, red, s, l, h, idx=None):
    """One unit against the oracle: every key (or the keys idx, for long units)."""
    from oracle import rkv_oracle as O
    spec = case.spec
    n = int(case.lens0[s])
    krows, _ = case.unit_rows(s, l, h)
    k = O.decode(krows, spec.dtype)
    got = red[row_of(spec, s, l, h)].cpu().numpy()
    assert np.all(np.isnan(got[n:])), f"unit ({s},{l},{h}): columns past N={n} written"
    if idx is None:
        ref, g = O.redundancy(k), got[:n].astype(np.float64)
    else:
        ref, g = O.redundancy_at(k, idx), got[np.asarray(idx)].astype(np.float64)
    tol = GRAM_REL * np.abs(ref).max() + GRAM_ABS
    err = np.abs(g - ref).max()
    assert err <= tol, f"unit ({s},{l},{h}) N={n}: redundancy off by {err:.3e} (tol {tol:.3e})"
    return err


def check_untriggered_rows(case, red):
    spec = case.spec
    for s in range(spec.num_seqs):
        if case.lens0[s] >= spec.budget + spec.buffer:
            continue
        for l in range(spec.num_layers):
            for h in range(spec.num_kv_heads):
                assert torch.isnan(red[row_of(spec, s, l, h)]).all(), f"untriggered ({s},{l},{h}) written"


CASES = {
    # several 256-row blocks and 64-key tiles, ragged tails, one sequence below the trigger
    "ragged-d128": syn.config(1).with_(name="g-ragged", seed=41, num_seqs=3, num_layers=2,
                                        num_q_heads=8, num_kv_heads=2, budget=256, buffer=32,
                                        lens=(777, 250, 300)),
    "d64-mha": syn.config(1).with_(name="g-d64", seed=42, num_seqs=2, num_layers=2, num_q_heads=4,
                                    num_kv_heads=4, head_dim=64, window=4, budget=200, buffer=40,
                                    lens=(513, 240)),
    # short units: N = 3 (the shortest this budget triggers), one partial tile, one row block
    "tiny-units": syn.config(1).with_(name="g-tiny", seed=43, num_seqs=3, num_layers=1,
                                       num_q_heads=2, num_kv_heads=2, window=1, budget=2, buffer=1,
                                       lens=(3, 65, 129)),
    "paged-bs16": syn.config(3).with_(name="g-p16", seed=44, num_seqs=3, num_layers=2,
                                       num_q_heads=8, num_kv_heads=2, budget=300, buffer=45,
                                       num_blocks=300, lens=(345, 500, 200)),
    "paged-bs1": syn.config(3).with_(name="g-p1", seed=45, num_seqs=2, num_layers=2, num_q_heads=8,
                                      num_kv_heads=2, budget=60, buffer=10, block_size=1,
                                      num_blocks=200, lens=(70, 90)),
    "paged-bs1024-d64": syn.config(3).with_(name="g-p1024", seed=46, num_seqs=2, num_layers=2,
                                            num_q_heads=4, num_kv_heads=2, head_dim=64,
                                            budget=1500, buffer=100, block_size=1024,
                                            num_blocks=8, lens=(1600, 2100)),
    "runs-dups": syn.config(4).with_(name="g-runs", seed=47, num_seqs=2, num_layers=1,
                                     lens=(1152, 1152)),
    # longest unit 1100 keys at head_dim 128: the 384-row workgroups (their last
    # block wastes 52 rows against the 256-row form's 180); units ending 2 and 1
    # rows into a block, one unit shorter than a block, one below the trigger
    "rows384-ragged": syn.config(1).with_(name="g-384", seed=51, num_seqs=4, num_layers=2,
                                           num_q_heads=8, num_kv_heads=2, budget=256, buffer=32,
                                           lens=(1100, 770, 385, 250)),
    "rows384-paged-bs16": syn.config(3).with_(name="g-384p", seed=52, num_seqs=3, num_layers=2,
                                               num_q_heads=8, num_kv_heads=2, budget=300,
                                               buffer=45, num_blocks=220, lens=(1100, 800, 350)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gram_small(name):
    spec = CASES[name]
    case = make_case(spec)
    red = run_gram(case)
    units = sample_units(spec, 10**9)
    worst = max(check_gram_unit(case, red, *u) for u in units)
    check_untriggered_rows(case, red)
    log(f"gram {name}: {len(units)} units match the oracle (max error {worst:.2e})")


def test_gram_zero_keys():
    """Zero keys have cosine 0 with every key (and redundancy 0)."""
    spec = syn.config(1).with_(name="g-zero", seed=48, num_seqs=1, num_layers=1, num_q_heads=4,
                               num_kv_heads=2, budget=200, buffer=20, lens=(300,))
    case = ContigCase(spec)
    zero = [0, 1, 63, 64, 127, 128, 299]
    case.k_host[:, :, :, zero] = 0
    case.k[:, :, :, zero] = 0
    red = run_gram(case)
    for h in range(spec.num_kv_heads):
        check_gram_unit(case, red, 0, 0, h)
        got = red[row_of(spec, 0, 0, h)].cpu().numpy()
        assert np.all(got[zero] == 0.0), "zero keys must have redundancy exactly 0"


def test_gram_matches_rank_one_scoring():
    """The Gram path and rkv_score's redundancy (rank-one form) agree on the
    Llama-8B-shaped step (256 units of 1152 keys); sampled units against the
    oracle at the Gram bar."""
    spec = syn.config(1)
    case = ContigCase(spec)
    red = run_gram(case, stride=1152)
    cfg = config_of(spec)
    n = 1152
    rows = spec.num_layers * spec.num_seqs * spec.num_kv_heads
    scores = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    red1 = torch.empty_like(scores)
    imp = torch.empty_like(scores)
    ws = torch.empty(max(256, B.rkv_workspace_size(cfg, 1, n)), dtype=torch.uint8, device="cuda")
    B.rkv_score(cfg, case.cache, case.q, 1, case.lens0.astype(np.int32), scores, n, imp, red1,
                ws, ws.numel())
    torch.cuda.synchronize()
    a, b = red.cpu().numpy().astype(np.float64), red1.cpu().numpy().astype(np.float64)
    for r in range(rows):
        tol = TOL * np.abs(b[r]).max()
        assert np.abs(a[r] - b[r]).max() <= tol, f"row {r}: Gram and rank-one redundancy differ"
    for u in sample_units(spec, 12, seed=5):
        check_gram_unit(case, red, *u)
    log(f"gram vs rank-one: {rows} rows agree; sampled units match the oracle")


def test_gram_max_length():
    """One unit at the longest accepted cache (RKV_MAX_LEN keys): sampled rows
    against the oracle's row-at-a-time definition."""
    n = B.RKV_MAX_LEN
    spec = syn.config(1).with_(name="g-max", seed=49, num_seqs=1, num_layers=1, num_q_heads=2,
                               num_kv_heads=1, budget=1000, buffer=100, lens=(n,))
    case = ContigCase(spec)
    red = run_gram(case, stride=n)
    idx = [0, 1, 127, 128, 4095, 16384, n - 65, n - 64, n - 2, n - 1]
    err = check_gram_unit(case, red, 0, 0, 0, idx=idx)
    got = red[0].cpu().numpy()
    assert np.all(np.isfinite(got)), "every row of the unit written"
    log(f"gram max length: N={n} sampled rows match the oracle (max error {err:.2e})")


def test_gram_many_sequences():
    """More triggered sequences than one launch's table holds (128): the call
    runs several launches; sequences of the second launch and untriggered
    ones in between are checked."""
    lens = tuple(70 if s % 7 else 50 for s in range(160))    # every 7th below the trigger
    spec = syn.config(1).with_(name="g-many", seed=50, num_seqs=160, num_layers=1, num_q_heads=2,
                               num_kv_heads=1, head_dim=64, window=2, budget=60, buffer=10,
                               lens=lens)
    case = ContigCase(spec)
    red = run_gram(case)
    trig = [s for s in range(spec.num_seqs) if lens[s] >= spec.budget + spec.buffer]
    assert len(trig) > 128
    for s in trig[:3] + trig[125:]:
        check_gram_unit(case, red, s, 0, 0)
    check_untriggered_rows(case, red)
    log(f"gram many sequences: {len(trig)} triggered, launches split at 128, sampled units match")
