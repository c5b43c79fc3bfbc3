"""The oracle comparisons of one unit, for worker processes of the GPU tests.

This module imports numpy and the CPU oracle only (no torch, no HIP library),
so processes that run it never open the GPU.  Its input is what
gpu_harness.unit_job_inputs gathers from the device: plain numpy arrays.
"""
import numpy as np

TOL = 1e-3    # scores: relative, fp32 accumulation against float64


def oracle_unit_job(job):
    """check_unit's comparisons for one unit, in a worker process (CPU only).
    Returns (keep differences inside the band, error message or None)."""
    from types import SimpleNamespace
    from oracle import rkv_oracle as O
    spec = SimpleNamespace(num_q_heads=job["hq"], num_kv_heads=job["hkv"], dtype=job["dtype"],
                           budget=job["budget"], window=job["window"], mix_lambda=job["lam"])
    o = O.step_unit(spec, job["q"], job["krows"], job["vrows"], job["h"])
    where, n, B_, w = job["where"], job["krows"].shape[0], job["budget"], job["window"]
    try:
        if job["imp"] is not None:
            err_i = np.abs(job["imp"].astype(np.float64) - o["imp"])
            assert np.all(err_i <= TOL * o["imp"]), f"{where}: importance off"
            tol_r = TOL * np.abs(o["red"]).max()
            assert np.abs(job["red"].astype(np.float64) - o["red"]).max() <= tol_r, f"{where}: redundancy off"
        tol_s = TOL * np.abs(o["score"]).max()
        err_s = np.abs(job["score"].astype(np.float64) - o["score"]).max()
        assert err_s <= tol_s, f"{where}: score off by {err_s:.3e} (tol {tol_s:.3e})"
        keep = job["keep"].astype(np.int64)
        same = O.select_keep(job["score"].astype(np.float64), n, B_, w)
        assert np.array_equal(keep, same), f"{where}: keep differs from the rule applied to GPU scores"
        diff = set(keep.tolist()) ^ set(o["keep"].tolist())
        if diff:
            t = np.sort(o["score"][: n - w])[::-1][B_ - w - 1]
            bad = [j for j in diff if abs(o["score"][j] - t) > tol_s]
            assert not bad, f"{where}: keep differs outside the band at {bad[:5]}"
        assert np.array_equal(job["gk"], O.compact_rows(job["krows"], keep)), f"{where}: compacted K differs"
        assert np.array_equal(job["gv"], O.compact_rows(job["vrows"], keep)), f"{where}: compacted V differs"
    except AssertionError as e:
        return 0, str(e)
    return len(diff), None


def run_jobs(jobs, workers=12):
    """oracle_unit_job over an iterable of jobs in `workers` spawned processes
    (fresh interpreters: nothing of the caller's GPU state is inherited), one
    BLAS thread each.  A worker that dies raises BrokenProcessPool rather than
    leaving the caller waiting.  Returns (total band differences, errors)."""
    import os
    from concurrent.futures import ProcessPoolExecutor
    from multiprocessing import get_context
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    for k in keys:
        os.environ[k] = "1"    # read by the workers' BLAS at start-up
    near, errors = 0, []
    try:
        with ProcessPoolExecutor(workers, mp_context=get_context("spawn")) as ex:
            for nb, err in ex.map(oracle_unit_job, jobs, chunksize=4):
                near += nb
                if err:
                    errors.append(err)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return near, errors
