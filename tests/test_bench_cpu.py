"""bench.py host logic on a machine without a GPU: the one-GPU rule, the
fused-launch predicate per workload, and the use of committed counter
summaries only while they match the kernel source."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

import rkv_synth as syn

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_fused_launch_predicate_per_workload():
    b = load_bench()
    expect = {0: False,    # fp32
              1: True,     # bf16, N 1152, G*w 32
              2: False,    # N 2176 > 1280
              3: False,    # N 4352
              4: True}     # bf16, N 1152, G*w 64
    for i, fused in expect.items():
        spec = syn.config(i)
        lens = syn.seq_lens(spec)
        trig = lens[lens >= spec.budget + spec.buffer]
        assert b.fused_launch(spec, trig) == fused, spec.name
    d64 = syn.config(1).with_(head_dim=64)
    assert b.fused_launch(d64, np.array([2560]))
    assert not b.fused_launch(d64, np.array([2561]))
    assert not b.fused_launch(syn.config(1), np.array([], dtype=np.int64))


def test_counter_summary_used_only_for_the_current_source(tmp_path, monkeypatch):
    b = load_bench()
    monkeypatch.setattr(b, "PROFILE_DIR", str(tmp_path))
    assert b.measured_traffic("step", "wl") is None            # no summary
    path = tmp_path / "step_wl_counters.txt"
    path.write_text(f"source_hash: {b.source_hash('step')}\nhbm_bytes_per_launch: 1234.5\n")
    assert b.measured_traffic("step", "wl") == 1234.5
    path.write_text("source_hash: 0000000000000000\nhbm_bytes_per_launch: 1234.5\n")
    assert b.measured_traffic("step", "wl") is None            # taken on other code


def test_source_hash_ignores_comments_only():
    b = load_bench()
    h = b.source_hash("select")
    assert len(h) == 16 and h == b.source_hash("select")
    assert b.source_hash("step") != b.source_hash("gram")


def test_committed_counter_summaries_name_a_kernel_and_workload():
    b = load_bench()
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.endswith("_counters.txt")]
    assert names
    for f in names:
        kernel = f.split("_", 1)[0]
        assert kernel in b.KERNEL_SOURCES, f
        text = open(os.path.join(prof, f)).read()
        assert "source_hash:" in text and "hbm_bytes_per_launch:" in text and "rocprofv3" in text, f


@pytest.mark.parametrize("argv", [["--steps", "0"], ["--warmup", "-1"]])
def test_bad_step_counts_are_rejected(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "must be" in r.stderr


def test_cpu_baseline_host_facts():
    """The CPU baseline names the host's CPU model and counts the threads the
    oracle may use (its BLAS pool within this process's CPU affinity)."""
    b = load_bench()
    assert 1 <= b.cpu_threads() <= len(os.sched_getaffinity(0))
    model = b.cpu_model()
    assert model and model != "unknown"
