"""The worker-pool form of the per-unit oracle comparison (used by the GPU
parity tests at full size), on the CPU: jobs built from the oracle's own
outputs pass; a planted difference in a compacted row, a score or a keep row
is reported; the pool runs in spawned processes under pytest."""
import numpy as np
import pytest

import oracle_jobs
import rkv_synth as syn
from oracle import rkv_oracle as O

pytestmark = pytest.mark.cpu


def job_from_oracle(seed):
    spec = syn.config(0).with_(seed=seed)
    k = syn.keys(spec, 0, 0)[0]
    v = syn.values(spec, 0, 0)[0]
    q = syn.build_queries(spec)[0, 0]
    o = O.step_unit(spec, q, k, v, 0)
    return dict(where=f"seed {seed}", dtype=spec.dtype, hq=spec.num_q_heads, hkv=spec.num_kv_heads,
                budget=spec.budget, window=spec.window, lam=spec.mix_lambda, h=0, q=q, krows=k,
                vrows=v, score=o["score"].astype(np.float32), keep=o["keep"].astype(np.int32),
                imp=o["imp"].astype(np.float32), red=o["red"].astype(np.float32),
                gk=O.compact_rows(k, o["keep"]), gv=O.compact_rows(v, o["keep"]))


def test_pool_passes_and_reports():
    good = [job_from_oracle(s) for s in range(6)]
    near, errors = oracle_jobs.run_jobs(good, workers=3)
    assert errors == []
    bad_rows = job_from_oracle(7)
    bad_rows["gv"] = bad_rows["gv"].copy()
    bad_rows["gv"][3, 5] += 1
    bad_score = job_from_oracle(8)
    bad_score["score"] = bad_score["score"] * 1.01
    bad_keep = job_from_oracle(9)
    bad_keep["keep"] = bad_keep["keep"].copy()
    bad_keep["keep"][0] += 1
    near, errors = oracle_jobs.run_jobs([bad_rows, bad_score, bad_keep] + good[:2], workers=2)
    assert len(errors) == 3
    assert "compacted V differs" in errors[0] and "score off" in errors[1] and "keep differs" in errors[2]
