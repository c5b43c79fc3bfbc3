"""Device-side helpers shared by the GPU tests and the benchmark.

Uploads seeded synthetic caches (rkv_synth) to the GPU, runs the three C ABI
calls through the binding, downloads results, and compares one unit at a
time with the CPU oracle.  The oracle is imported lazily and only by the
comparison helpers.
"""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import rkv_synth as syn
from kv_cache_compression_decode_amd import binding as B
from kv_cache_compression_decode_amd.step import RKVStep

TOL = 1e-3    # scores: relative, fp32 accumulation against float64


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def config_of(spec: syn.Spec, shared: bool = False) -> B.rkv_config:
    return B.make_config(spec.num_layers, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                         spec.budget, spec.buffer, spec.window, spec.mix_lambda, spec.dtype,
                         spec.layout, spec.block_size, shared_selection=shared)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if dtype == "bf16" else a


def canary_value(spec):
    if spec.dtype == "bf16":
        return int(np.int16(np.uint16(syn.CANARY_BF16).view(np.int16)))
    return float(syn.CANARY_F32)


def torch_storage_dtype(spec):
    return torch.int16 if spec.dtype == "bf16" else torch.float32


class ContigCase:
    """Contiguous K, V (L, S, Hkv, cap, d) and window queries on the device."""

    def __init__(self, spec: syn.Spec, capacity=None, device="cuda", keep_host=True):
        self.spec = spec
        self.lens0 = syn.seq_lens(spec)
        self.cap = int(self.lens0.max()) if capacity is None else capacity
        k, v = syn.build_contiguous(spec, self.cap)
        q = syn.build_queries(spec)
        self.k, self.v, self.q = to_dev(k, device), to_dev(v, device), to_dev(q, device)
        self.k_host, self.v_host, self.q_host = (k, v, q) if keep_host else (None, None, q)
        self.cache = B.make_cache(self.k, self.v, capacity=self.cap)
        self.free_capacity = 0

    def unit_rows(self, s, l, h):
        n = int(self.lens0[s])
        return self.k_host[l, s, h, :n], self.v_host[l, s, h, :n]

    def gpu_rows(self, s, l, h, count):
        return (to_host(self.k[l, s, h, :count], self.spec.dtype),
                to_host(self.v[l, s, h, :count], self.spec.dtype))


class PagedCase:
    """Paged pools (L, nblk, Hkv, bs, d) filled with the canary, referenced
    blocks uploaded chunk by chunk, and the block table on the device."""

    def __init__(self, spec: syn.Spec, device="cuda"):
        self.spec = spec
        self.lens0 = syn.seq_lens(spec)
        self.bt = syn.block_table(spec)
        L, nb, hk, bs, d = (spec.num_layers, spec.num_blocks, spec.num_kv_heads,
                            spec.block_size, spec.head_dim)
        dt = torch_storage_dtype(spec)
        self.k = torch.empty((L, nb, hk, bs, d), dtype=dt, device=device)
        self.v = torch.empty_like(self.k)
        self.k.fill_(canary_value(spec))
        self.v.fill_(canary_value(spec))
        self.bt_dev = torch.from_numpy(self.bt).to(device)
        self.plans = [syn.dup_plan(spec, s, int(self.lens0[s])) for s in range(spec.num_seqs)]
        self.q_host = syn.build_queries(spec)
        self.q = to_dev(self.q_host, device)

        def gen(sl):
            s, l = sl
            n = int(self.lens0[s])
            return s, l, syn.keys(spec, s, l, n, self.plans[s]), syn.values(spec, s, l, n)

        jobs = [(s, l) for l in range(L) for s in range(spec.num_seqs)]
        with ThreadPoolExecutor(min(16, len(jobs))) as ex:
            for s, l, kc, vc in ex.map(gen, jobs):
                self._upload(self.k, l, s, kc)
                self._upload(self.v, l, s, vc)
        self.cache = B.make_cache(self.k, self.v, num_blocks=nb, block_table=self.bt_dev,
                                  max_blocks_per_seq=self.bt.shape[1])
        bsz = spec.block_size
        kept = -(-spec.budget // bsz)
        self.free_capacity = int(sum(max(0, -(-int(n) // bsz) - kept)
                                     for n in self.lens0 if n >= spec.budget + spec.buffer))

    def _upload(self, pool, l, s, chunk):
        spec = self.spec
        hk, n, d = chunk.shape
        bs = spec.block_size
        nb = -(-n // bs)
        pad = nb * bs - n
        if pad:
            fill = np.full((hk, pad, d), syn.CANARY_BF16 if spec.dtype == "bf16" else syn.CANARY_F32,
                           dtype=chunk.dtype)
            chunk = np.concatenate([chunk, fill], axis=1)
        blocks = chunk.reshape(hk, nb, bs, d).transpose(1, 0, 2, 3)
        idx = torch.from_numpy(self.bt[s, :nb].astype(np.int64)).to(pool.device)
        pool[l].index_copy_(0, idx, to_dev(np.ascontiguousarray(blocks), pool.device))

    def unit_rows(self, s, l, h):
        n = int(self.lens0[s])
        return (syn.keys(self.spec, s, l, n, self.plans[s])[h],
                syn.values(self.spec, s, l, n)[h])

    def gpu_rows(self, s, l, h, count):
        bs = self.spec.block_size
        nb = -(-count // bs)
        idx = self.bt_dev[s, :nb].long()
        kk = self.k[l].index_select(0, idx)[:, h].reshape(nb * bs, -1)[:count]
        vv = self.v[l].index_select(0, idx)[:, h].reshape(nb * bs, -1)[:count]
        return to_host(kk, self.spec.dtype), to_host(vv, self.spec.dtype)


def make_case(spec: syn.Spec, **kw):
    return PagedCase(spec, **kw) if spec.layout == "paged" else ContigCase(spec, **kw)


def run_step(case, keep_parts=True, sentinel=True, shared=False, fused=False):
    """Run score, select, compact on the case (fused: the single rkv_step
    call, which writes no importance / redundancy); returns (RKVStep, lens
    after)."""
    spec = case.spec
    cfg = config_of(spec, shared)
    maxn = int(case.lens0.max())
    step = RKVStep(cfg, spec.num_seqs, maxn, keep_parts=keep_parts and not fused,
                   free_capacity=case.free_capacity)
    if sentinel:   # rows of untriggered units must stay as they are
        step.scores.fill_(float("nan"))
        step.keep.fill_(-7)
        if step.importance is not None:
            step.importance.fill_(float("nan"))
            step.redundancy.fill_(float("nan"))
    lens = case.lens0.astype(np.int32).copy()
    (step.fused if fused else step)(case.cache, case.q, lens)
    torch.cuda.synchronize()
    return step, lens


def unit_outputs(step, spec, s, l, h, n):
    maxn = step.max_len
    row = (l * spec.num_seqs + s) * spec.num_kv_heads + h
    out = {"score": step.scores[row * maxn: row * maxn + n].cpu().numpy(),
           "keep": step.keep[row * spec.budget:(row + 1) * spec.budget].cpu().numpy()}
    if step.importance is not None:
        out["imp"] = step.importance[row * maxn: row * maxn + n].cpu().numpy()
        out["red"] = step.redundancy[row * maxn: row * maxn + n].cpu().numpy()
    return out


def check_unit(case, step, s, l, h, tag=""):
    """GPU outputs of one unit against the oracle: scores within tolerance,
    keep set exact given the GPU's own scores and within the threshold band
    of the oracle's, compacted rows bit-exact given the GPU's keep set."""
    from oracle import rkv_oracle as O
    spec = case.spec
    n = int(case.lens0[s])
    krows, vrows = case.unit_rows(s, l, h)
    o = O.step_unit(spec, case.q_host[l, s], krows, vrows, h)
    g = unit_outputs(step, spec, s, l, h, n)
    where = f"{tag} unit (s={s}, l={l}, h={h}) N={n}"
    B_, w = spec.budget, spec.window
    if "imp" in g:
        err_i = np.abs(g["imp"].astype(np.float64) - o["imp"])
        assert np.all(err_i <= TOL * o["imp"]), f"{where}: importance off by {np.max(err_i / o['imp']):.3e} rel"
        tol_r = TOL * np.abs(o["red"]).max()
        err_r = np.abs(g["red"].astype(np.float64) - o["red"]).max()
        assert err_r <= tol_r, f"{where}: redundancy off by {err_r:.3e} (tol {tol_r:.3e})"
    tol_s = TOL * np.abs(o["score"]).max()
    err_s = np.abs(g["score"].astype(np.float64) - o["score"]).max()
    assert err_s <= tol_s, f"{where}: score off by {err_s:.3e} (tol {tol_s:.3e})"
    keep = g["keep"].astype(np.int64)
    # the same decision in the same precision: the oracle's rule on the GPU's fp32 scores
    same = O.select_keep(g["score"].astype(np.float64), n, B_, w)
    assert np.array_equal(keep, same), f"{where}: keep differs from the rule applied to GPU scores"
    # against the float64 oracle: differences only inside the threshold band
    diff = set(keep.tolist()) ^ set(o["keep"].tolist())
    if diff:
        cand = np.sort(o["score"][: n - w])[::-1]
        t = cand[B_ - w - 1]
        bad = [j for j in diff if abs(o["score"][j] - t) > tol_s]
        assert not bad, f"{where}: keep differs outside the band at {bad[:5]}"
    gk, gv = case.gpu_rows(s, l, h, B_)
    assert np.array_equal(gk, O.compact_rows(krows, keep)), f"{where}: compacted K differs"
    assert np.array_equal(gv, O.compact_rows(vrows, keep)), f"{where}: compacted V differs"
    return len(diff)


def unit_job_inputs(case, step, s, l, h):
    """Everything check_unit compares, as plain numpy arrays (for a worker)."""
    spec = case.spec
    n = int(case.lens0[s])
    krows, vrows = case.unit_rows(s, l, h)
    g = unit_outputs(step, spec, s, l, h, n)
    gk, gv = case.gpu_rows(s, l, h, spec.budget)
    return dict(where=f"unit (s={s}, l={l}, h={h}) N={n}", dtype=spec.dtype,
                hq=spec.num_q_heads, hkv=spec.num_kv_heads, budget=spec.budget,
                window=spec.window, lam=spec.mix_lambda, h=h, q=case.q_host[l, s],
                krows=np.ascontiguousarray(krows), vrows=np.ascontiguousarray(vrows),
                score=g["score"], keep=g["keep"], imp=g.get("imp"), red=g.get("red"), gk=gk, gv=gv)


def check_units_parallel(case, step, units, tag, workers=12):
    """check_unit for many units, the oracle in worker processes that import
    numpy and the oracle only (oracle_jobs.run_jobs); inputs gathered here."""
    import oracle_jobs
    jobs = (unit_job_inputs(case, step, s, l, h) for (s, l, h) in units)
    near, errors = oracle_jobs.run_jobs(jobs, workers)
    assert not errors, f"{tag}: {len(errors)} units differ, first: {errors[0]}"
    log(f"{tag}: {len(units)} units match the oracle ({near} keep differences inside the band)")
    return near


def one_unit_per_layer(spec, seed=0, triggered=None):
    """One (sequence, layer) pair's unit for every triggered sequence and
    layer, the kv head drawn at random."""
    lens = syn.seq_lens(spec)
    rng = np.random.default_rng([992, seed])
    return [(s, l, int(rng.integers(spec.num_kv_heads)))
            for s in range(spec.num_seqs) if lens[s] >= spec.budget + spec.buffer
            and (triggered is None or s in triggered) for l in range(spec.num_layers)]


def keep_invariants_on_device(step, spec, lens):
    """Every triggered unit's keep row: budget entries, strictly ascending,
    inside [0, N), the window last (checked on the GPU for all units)."""
    B_, w = spec.budget, spec.window
    keep = step.keep.view(spec.num_layers, spec.num_seqs, spec.num_kv_heads, B_).long()
    count = 0
    for s in range(spec.num_seqs):
        n = int(lens[s])
        if n < spec.budget + spec.buffer:
            continue
        ks = keep[:, s]
        assert bool((ks[..., 1:] > ks[..., :-1]).all()), f"seq {s}: a keep row is not ascending"
        assert bool((ks[..., 0] >= 0).all()) and bool((ks[..., -1] == n - 1).all())
        win = torch.arange(n - w, n, device=ks.device)
        assert bool((ks[..., B_ - w:] == win).all()), f"seq {s}: the window is not kept last"
        assert bool((ks[..., B_ - w - 1] < n - w).all())
        count += spec.num_layers * spec.num_kv_heads
    return count


def check_layer_shared(case, step, s, l, tag=""):
    """Head-shared selection for one (sequence, layer): every head's scores
    within tolerance of the oracle; one keep row shared by all heads, equal to
    the oracle's rule applied to the float32 sum of the GPU's scores (head 0
    first, the kernel's order) and to the float64 oracle's shared set outside
    the threshold band; every head's compacted rows bit-exact."""
    from oracle import rkv_oracle as O
    spec = case.spec
    n = int(case.lens0[s])
    B_, w, H = spec.budget, spec.window, spec.num_kv_heads
    where = f"{tag} layer (s={s}, l={l}) N={n}"
    ref, rows, gsc, keeps, tols = [], [], [], [], []
    for h in range(H):
        krows, vrows = case.unit_rows(s, l, h)
        o = O.step_unit(spec, case.q_host[l, s], krows, vrows, h)
        g = unit_outputs(step, spec, s, l, h, n)
        tol_s = TOL * np.abs(o["score"]).max()
        err_s = np.abs(g["score"].astype(np.float64) - o["score"]).max()
        assert err_s <= tol_s, f"{where} head {h}: score off by {err_s:.3e} (tol {tol_s:.3e})"
        ref.append(o["score"])
        rows.append((krows, vrows))
        gsc.append(g["score"].astype(np.float32))
        keeps.append(g["keep"].astype(np.int64))
        tols.append(tol_s)
    keep = keeps[0]
    for h in range(1, H):
        assert np.array_equal(keeps[h], keep), f"{where}: head {h} keeps a different set"
    acc = gsc[0].copy()
    for h in range(1, H):
        acc = (acc + gsc[h]).astype(np.float32)
    same = O.select_keep(acc.astype(np.float64), n, B_, w)
    assert np.array_equal(keep, same), f"{where}: keep differs from the rule on the summed GPU scores"
    total = O.shared_score(np.stack(ref))
    diff = set(keep.tolist()) ^ set(O.select_keep_shared(np.stack(ref), n, B_, w).tolist())
    if diff:
        t = np.sort(total[: n - w])[::-1][B_ - w - 1]
        band = float(np.sum(tols))
        bad = [j for j in diff if abs(total[j] - t) > band]
        assert not bad, f"{where}: keep differs outside the band at {bad[:5]}"
    for h in range(H):
        gk, gv = case.gpu_rows(s, l, h, B_)
        assert np.array_equal(gk, O.compact_rows(rows[h][0], keep)), f"{where} head {h}: K differs"
        assert np.array_equal(gv, O.compact_rows(rows[h][1], keep)), f"{where} head {h}: V differs"
    return len(diff)


def sample_units(spec, count, seed=0, triggered=None):
    lens = syn.seq_lens(spec)
    trig = [s for s in range(spec.num_seqs) if lens[s] >= spec.budget + spec.buffer]
    if triggered is not None:
        trig = [s for s in trig if s in triggered]
    all_units = [(s, l, h) for s in trig for l in range(spec.num_layers)
                 for h in range(spec.num_kv_heads)]
    if len(all_units) <= count:
        return all_units
    rng = np.random.default_rng([991, seed])
    pick = rng.choice(len(all_units), size=count, replace=False)
    # always include the first and last unit
    pick = sorted(set(pick.tolist()) | {0, len(all_units) - 1})
    return [all_units[i] for i in pick]
