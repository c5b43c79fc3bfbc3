"""bench.py end to end on the GPU, briefly: one JSON line on stdout with the
fields and units the benchmark promises (the step's roofline object and the
oracle's CPU baseline included)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--cpu-seconds", "1"], capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool),
                     ("scaling", str), ("dtype", str), ("data", str), ("config", dict),
                     ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), (key, d[key])
    assert d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "steps/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "llama8b-1seq"
    # rates: one 1152-token sequence per step, scored on 32 layers x 8 kv heads
    assert abs(d["cache_tokens_per_s"] - d["value"] * 1152) <= 1e-3 * d["cache_tokens_per_s"]
    assert abs(d["tokens_scored_per_s"] - d["cache_tokens_per_s"] * 32 * 8) <= 1e-3 * d["tokens_scored_per_s"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_bench_device_lens_line():
    """--device-lens times rkv_step_device (trigger table built on the GPU);
    bench.py itself checks every step's device lengths afterwards."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--cpu-seconds", "0", "--device-lens"], capture_output=True, text=True,
                       timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    assert d["entry"] == "rkv_step_device" and d["value"] > 0 and d["steps"] == 3
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["achieved"] > 0
