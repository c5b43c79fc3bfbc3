"""The selection kernel (rkv_select) on crafted score rows: ties, signed
zeros, infinities, scores one ulp apart, a single eviction and the longest
cache, each against the oracle's keep set (exact: integer output)."""
import numpy as np
import pytest
import torch

from kv_cache_compression_decode_amd import binding as B

pytestmark = pytest.mark.gpu

F32 = np.float32


def scores_for(kind: str, n: int, rng) -> np.ndarray:
    if kind == "all-equal":
        return np.full(n, 0.25, F32)
    if kind == "two-values":
        return rng.integers(0, 2, n).astype(F32)
    if kind == "signed-zeros":
        return rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], F32), n)
    if kind == "infinities":
        s = rng.normal(0, 1, n).astype(F32)
        s[rng.choice(n, n // 10, replace=False)] = np.inf
        s[rng.choice(n, n // 10, replace=False)] = -np.inf
        return s
    if kind == "one-ulp":   # every key shares its leading bits
        return (np.float32(1.0) + rng.integers(0, 64, n).astype(F32) * np.finfo(F32).eps).astype(F32)
    if kind == "mixed-sign":
        return rng.normal(0, 1e3, n).astype(F32)
    if kind == "ascending":
        return np.arange(n, dtype=F32)
    if kind == "descending":
        return -np.arange(n, dtype=F32)
    return rng.normal(-0.18, 0.03, n).astype(F32)   # the spread of real unit scores


def run_select(scores: np.ndarray, n: int, budget: int, buffer: int, window: int) -> np.ndarray:
    cfg = B.make_config(1, 4, 1, 128, budget, buffer, window, 0.1)
    assert B.rkv_is_triggered(cfg, n)
    s = torch.from_numpy(scores).cuda()
    keep = torch.full((budget,), -1, dtype=torch.int32, device="cuda")
    B.rkv_select(cfg, 1, np.array([n], np.int32), s, n, keep)
    torch.cuda.synchronize()
    return keep.cpu().numpy()


KINDS = ["all-equal", "two-values", "signed-zeros", "infinities", "one-ulp", "mixed-sign",
         "ascending", "descending", "normal"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n,budget,buffer", [(1152, 1024, 128), (1001, 1000, 1), (200, 20, 180)])
def test_select_crafted(kind, n, budget, buffer):
    from oracle import rkv_oracle as O
    rng = np.random.default_rng(KINDS.index(kind) * 100003 + n)
    s = scores_for(kind, n, rng)
    got = run_select(s, n, budget, buffer, 8)
    want = O.select_keep(s.astype(np.float64), n, budget, 8)
    assert np.array_equal(got, want), (kind, n, np.flatnonzero(got != want)[:8])


def test_select_longest_cache():
    from oracle import rkv_oracle as O
    n = B.RKV_MAX_LEN
    rng = np.random.default_rng(7)
    for kind in ("normal", "two-values"):
        s = scores_for(kind, n, rng)
        got = run_select(s, n, 1024, n - 1024, 8)
        assert np.array_equal(got, O.select_keep(s.astype(np.float64), n, 1024, 8)), kind


@pytest.mark.parametrize("frac", [0.1, 1.0])
@pytest.mark.parametrize("n,budget,buffer", [(1152, 1024, 128), (200, 20, 180), (4352, 4096, 256)])
def test_select_nan_scores_give_a_valid_set(frac, n, budget, buffer):
    """NaN scores: the set is unspecified, but it must be a valid keep row --
    budget entries, strictly ascending, in range, the window at the end."""
    rng = np.random.default_rng([int(frac * 10), n])
    s = rng.normal(0, 1, n).astype(F32)
    s[rng.choice(n, int(frac * n), replace=False)] = np.nan
    w = 8
    got = run_select(s, n, budget, buffer, w)
    assert got.shape == (budget,)
    assert np.all(np.diff(got) > 0), "not strictly ascending"
    assert got[0] >= 0 and got[-1] == n - 1
    assert np.array_equal(got[budget - w:], np.arange(n - w, n)), "window not kept"
    assert np.all(got[: budget - w] < n - w)
