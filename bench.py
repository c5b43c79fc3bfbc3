"""Benchmark of the R-KV compression step on one MI355X.

One step = score, select and compact over one batch (all layers, all
triggered units) through the C ABI's rkv_step (for this workload one fused
kernel per launch; --three-calls times rkv_score + rkv_select + rkv_compact
instead), inputs already resident in HBM.
Compaction is in place, so every step gets its own pristine copy of the
cache, prepared before the timed region.

Prints one JSON line.  Defaults: the Llama-8B-shaped single-sequence
workload (32 layers, 32 q / 8 kv heads, d 128, bf16, N 1152, budget 1024,
buffer 128, window 8, lambda 0.1), 100 timed steps after 3 warm-up steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "compression steps/sec (cached tokens scored/s) at 1 GPU; % MFMA / % HBM roofline"
HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "step": ["rkv_step_impl.h", "rkv_unit_impl.h", "rkv_select_impl.h", "rkv_score_impl.h",
             "rkv_device.h", "rkv_launch.h"],
    "compact": ["rkv_compact.hip", "rkv_device.h", "rkv_launch.h"],
    "score": ["rkv_unit_impl.h", "rkv_long_impl.h", "rkv_score_impl.h", "rkv_device.h",
              "rkv_launch.h"],
    "select": ["rkv_select.hip", "rkv_select_impl.h", "rkv_device.h", "rkv_launch.h"],
    "gram": ["rkv_gram.hip", "rkv_score_impl.h", "rkv_device.h", "rkv_launch.h"],
    "kara": ["rkv_kara.hip", "rkv_kara.h", "rkv_score_impl.h", "rkv_select_impl.h", "rkv_device.h",
             "rkv_launch.h"],
}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of one MI355X


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: up to 100, as many pristine cache copies as fit in 40 GB)")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=1, help="workload index (0-4)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of the CPU-baseline sample (0 skips it)")
    p.add_argument("--device-lens", action="store_true",
                   help="time rkv_step_device (lengths in device memory, the trigger table built "
                        "by a kernel: the form a captured decode graph uses) instead of rkv_step")
    p.add_argument("--three-calls", action="store_true",
                   help="time rkv_score + rkv_select + rkv_compact instead of rkv_step")
    p.add_argument("--shared", action="store_true",
                   help="head-shared selection (one keep set per sequence and layer; three kernels)")
    p.add_argument("--gram", action="store_true",
                   help="time rkv_redundancy_gram (the explicit cosine Gram on the matrix cores) instead")
    p.add_argument("--kara", action="store_true",
                   help="time rkv_kara_step, the KARA-style window step (window 128 -> keep 32, "
                        "4 anchors of radius 2), on the workload's shape")
    p.add_argument("--window-store", action="store_true",
                   help="time rkv_window_store (one decode step's queries, all layers, into the ring)")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the timed region, one 256 MiB device copy (counter calibration)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the records measured after the timed region (the Gram on the matrix "
                        "cores, the three calls kernel by kernel, the streaming peaks)")
    args = p.parse_args()
    if args.steps is not None and args.steps < 1:
        p.error("--steps must be >= 1")
    if args.warmup < 0:
        p.error("--warmup must be >= 0")
    return args


def fused_launch(spec, trig_lens) -> bool:
    """Whether rkv_step runs one fused kernel for this batch (the condition
    include/rkv.h states: bf16, every unit up to 1280 keys at head_dim 128 or
    2560 at 64, and num_q_heads / num_kv_heads * window <= 78)."""
    nmax = 1280 if spec.head_dim == 128 else 2560
    return (spec.dtype == "bf16" and len(trig_lens) > 0 and int(max(trig_lens)) <= nmax
            and spec.group * spec.window <= 78)


def source_hash(kernel: str) -> str:
    """Hash of the kernel's source code with comments and whitespace removed
    (an edit to a comment leaves the compiled kernel, and so the counters
    taken on it, as they were)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kv_cache_compression_decode_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source for this workload; else None."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_hash:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(kernel):
        return None
    return float(m_bytes.group(1))


def cpu_threads() -> int:
    """Threads the oracle can run on: its BLAS pool, bounded by the cores this
    process may use (its CPU affinity)."""
    usable = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    return max(1, min(usable, blas))


def cpu_baseline(spec, case, seconds: float):
    """The oracle, as it stands, on this host's cores: units of the same
    workload, three samples of seconds / 3 each; the median sample's rate,
    reported as steps/s."""
    from oracle import rkv_oracle as O
    cores = cpu_threads()
    units = [(s, l, h) for s in range(spec.num_seqs) for l in range(spec.num_layers)
             for h in range(spec.num_kv_heads)
             if case.lens0[s] >= spec.budget + spec.buffer]
    def sample(budget):
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:
            s, l, h = units[done % len(units)]
            kr, vr = case.unit_rows(s, l, h)
            O.step_unit(spec, case.q_host[l, s], kr, vr, h)
            done += 1
        return done, time.perf_counter() - t0

    runs = sorted((done / dt, done, dt) for done, dt in (sample(seconds / 3) for _ in range(3)))
    rate, done, dt = runs[1]
    steps_per_s = rate / len(units)
    out = {"value": round(steps_per_s, 4), "unit": "steps/s", "cores": cores, "kind": "oracle",
           "cpu": cpu_model(), "cores_usable": len(os.sched_getaffinity(0)),
           "samples_steps_per_s": [round(r[0] / len(units), 4) for r in runs],
           "sample": f"median of 3 samples of {seconds / 3:.1f} s: {done} of the step's "
                     f"{len(units)} units in {dt:.1f} s (float64 numpy, explicit N x N Gram); "
                     f"value = units/s / units per step"}
    try:   # the same oracle on one thread, a third of the time budget
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1, t1 = sample(seconds / 3)
        out["value_1thread"] = round(d1 / t1 / len(units), 4)
        out["sample_1thread"] = f"{d1} units, {t1:.1f} s, one BLAS thread"
    except Exception:  # noqa: BLE001 - the single-thread figure is optional context
        pass
    return out


def cpu_model() -> str:
    """The CPU model name as lscpu gives it (else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_peaks(torch, stream) -> dict:
    """HBM bandwidth of this repository's streaming kernels (librkv_membench.so:
    16-byte accesses, each workgroup a contiguous stretch, eight loads in
    flight per lane) on 2 GiB buffers, eight times the 256 MB last-level
    cache: a read of every byte, and a copy (bytes read + bytes written).
    Best over launch sizes of 4, 8 and 16 workgroups per compute unit and
    five repetitions each."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_compression_decode_amd", "librkv_membench.so"))
    lib.rkv_membench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
    lib.rkv_membench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int32, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    nbytes = 2 << 30
    a = torch.full((nbytes,), 7, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = {}
    for name, moved in (("read", 1), ("copy", 2)):
        best = None
        for per_cu in (4, 8, 16):
            for rep in range(6):
                ev[0].record(stream)
                if name == "read":
                    rc = lib.rkv_membench_read(a.data_ptr(), nbytes, sink.data_ptr(), cus * per_cu,
                                               stream.cuda_stream)
                else:
                    rc = lib.rkv_membench_copy(b.data_ptr(), a.data_ptr(), nbytes, cus * per_cu,
                                               stream.cuda_stream)
                ev[1].record(stream)
                if rc != 0:
                    raise RuntimeError(f"rkv_membench_{name}: {rc}")
                torch.cuda.synchronize()
                if rep == 0:
                    continue   # the first launch of a shape warms up
                t = ev[0].elapsed_time(ev[1]) * 1e-3
                if best is None or t < best[0]:
                    best = (t, per_cu)
        out[f"hbm_stream_{name}_GBps"] = round(moved * nbytes / best[0] / 1e9, 1)
        out[f"hbm_stream_{name}_workgroups_per_cu"] = best[1]
    del a, b
    torch.cuda.synchronize()
    return out


def measured_peaks(torch, stream) -> dict:
    """Achievable peaks measured on this GPU, next to the spec figures: the
    streaming kernels above; a 1 GiB device-to-device copy by the runtime
    (read + write bytes / time); and an 8192^3 bf16 matrix product through
    torch (the vendor GEMM library) for the matrix cores.  Best of five timed
    repetitions each."""
    dev = torch.device("cuda:0")
    out = stream_peaks(torch, stream)
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    b.copy_(a)
    best = None
    for _ in range(5):
        ev[0].record(stream)
        b.copy_(a)
        ev[1].record(stream)
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[1]) * 1e-3
        best = t if best is None else min(best, t)
    out["hbm_copy_GBps"] = round(2 * a.numel() / best / 1e9, 1)
    del a, b
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    y = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    z = torch.matmul(x, y)
    best = None
    for _ in range(5):
        ev[0].record(stream)
        torch.matmul(x, y, out=z)
        ev[1].record(stream)
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[1]) * 1e-3
        best = t if best is None else min(best, t)
    out["bf16_gemm_TFLOPs"] = round(2.0 * n ** 3 / best / 1e12, 1)
    del x, y, z
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the step shards by sequence / layer / kv head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import rkv_synth as syn
    from gpu_harness import ContigCase, PagedCase, config_of
    from kv_cache_compression_decode_amd import binding as B
    from kv_cache_compression_decode_amd.step import RKVStep

    spec = syn.config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.window_store:
        return window_store_bench(args, spec)
    case = PagedCase(spec) if spec.layout == "paged" else ContigCase(spec)
    if args.gram:
        return gram_bench(args, spec, case)
    if args.kara:
        return kara_bench(args, spec, case)
    cfg = config_of(spec, shared=args.shared)
    copy_bytes = case.k.numel() * case.k.element_size() * 2
    # Paged pools too large to copy once per step (the 8-sequence paged workload
    # holds 137 GB of pools): one working pool, and before each step the blocks
    # the block table references are written back from a pristine copy of just
    # those blocks, outside the step's own timed interval.
    restore = spec.layout == "paged" and copy_bytes > (20 << 30)
    if args.steps is None:
        args.steps = 10 if restore else int(max(5, min(100, (40 << 30) // copy_bytes - args.warmup)))
    nsteps = args.warmup + args.steps
    lens0 = case.lens0.astype(np.int32)
    maxn = int(lens0.max())
    trig = lens0 >= spec.budget + spec.buffer
    units = int(trig.sum()) * spec.num_layers * spec.num_kv_heads
    step = RKVStep(cfg, spec.num_seqs, maxn, free_capacity=case.free_capacity)
    stream = torch.cuda.current_stream()

    # one pristine cache copy per step, prepared before timing
    if restore:
        ref = torch.from_numpy(np.unique(case.bt).astype(np.int64)).to(dev)
        pristine = (case.k.index_select(1, ref), case.v.index_select(1, ref))
        copies = [(case.k, case.v)] * nsteps
    else:
        copies = [(case.k.clone(), case.v.clone()) for _ in range(nsteps)]
    caches = []
    for kc, vc in copies:
        if spec.layout == "paged":
            caches.append(B.make_cache(kc, vc, num_blocks=spec.num_blocks, block_table=case.bt_dev,
                                       max_blocks_per_seq=case.bt.shape[1]))
        else:
            caches.append(B.make_cache(kc, vc, capacity=case.cap))
    lens_per = [lens0.copy() for _ in range(nsteps)]
    if args.device_lens:
        if restore or args.three_calls:
            raise SystemExit("--device-lens times rkv_step_device alone, on workloads whose caches "
                             "are copied per step")
        d_lens_per = [torch.from_numpy(lens0.copy()).to(dev) for _ in range(nsteps)]
    # --three-calls: events around each of the three kernels (a breakdown;
    # the markers themselves add GPU time between launches).  rkv_step: one
    # event pair around the whole timed region, so nothing runs between the
    # back-to-back launches and region time / steps is the launch duration.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nsteps)]
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()

    def run(i):
        if restore:   # untimed: the referenced blocks back to their pristine contents
            case.k.index_copy_(1, ref, pristine[0])
            case.v.index_copy_(1, ref, pristine[1])
            ev[i][0].record(stream)
            if args.three_calls:
                step.score(caches[i], case.q, lens_per[i], stream)
                ev[i][1].record(stream)
                step.select(lens_per[i], stream)
                ev[i][2].record(stream)
                step.compact(caches[i], lens_per[i], stream)
            else:
                step.fused(caches[i], case.q, lens_per[i], stream)
            ev[i][3].record(stream)
        elif args.three_calls:
            e = ev[i]
            e[0].record(stream)
            step.score(caches[i], case.q, lens_per[i], stream)
            e[1].record(stream)
            step.select(lens_per[i], stream)
            e[2].record(stream)
            step.compact(caches[i], lens_per[i], stream)
            e[3].record(stream)
        elif args.device_lens:
            step.device(caches[i], case.q, d_lens_per[i], stream)
        else:
            step.fused(caches[i], case.q, lens_per[i], stream)

    if args.device_lens:   # workspace and free counts allocated outside the timed region
        step.device(caches[0], case.q, torch.from_numpy(lens0.copy()).to(dev), stream)
        copies[0][0].copy_(case.k)   # copy 0 back to its pristine contents
        copies[0][1].copy_(case.v)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.warmup, nsteps):
        run(i)
    region[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    # rows the compaction actually moves (keep[i] != i), from the last step's keep
    # lists of the triggered units (every step sees the same inputs; rows of
    # other sequences are never written)
    keep = step.keep.view(spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.budget)
    keep = keep.cpu().numpy()[:, trig].reshape(-1, spec.budget)
    moved_rows = int((keep != np.arange(spec.budget)[None, :]).sum()) if units else 0
    if args.device_lens:   # every step left the compacted lengths in its device tensor
        want = np.where(trig, spec.budget, lens0).astype(np.int32)
        for i, d in enumerate(d_lens_per):
            if not np.array_equal(d.cpu().numpy(), want):
                raise RuntimeError(f"rkv_step_device step {i}: device lengths {d.cpu().numpy()} != {want}")

    ms = (t1 - t0) * 1e3 / args.steps
    region_us = region[0].elapsed_time(region[1]) * 1e3 / args.steps
    timed = ev[args.warmup:]
    if restore:   # the wall clock includes the untimed restores: the step is the event interval
        ms = sum(e[0].elapsed_time(e[3]) for e in timed) / len(timed)
        region_us = ms * 1e3

    def avg_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in timed) / len(timed)

    esz = 2 if spec.dtype == "bf16" else 4
    row = spec.head_dim * esz
    gw = spec.group * spec.window
    tokens = int(sum(int(n) for n in lens0[trig])) * spec.num_layers * spec.num_kv_heads
    # algorithmic bytes per launch, per unit: read K once, read the window
    # queries, write S and the keep list; compaction: moved rows (keep[i] != i)
    # of K and V, each read and written once
    q_bytes = units * gw * row
    score_bytes = tokens * row + q_bytes + tokens * 4
    select_bytes = tokens * 4 + units * spec.budget * 4
    compact_bytes = moved_rows * row * 2 * 2 + units * spec.budget * 4 * 2
    if args.three_calls:
        kern = {"score": {"us": avg_ms(0, 1) * 1e3, "bytes": score_bytes},
                "select": {"us": avg_ms(1, 2) * 1e3, "bytes": select_bytes},
                "compact": {"us": avg_ms(2, 3) * 1e3, "bytes": compact_bytes}}
    else:
        # the fused kernel holds the keys on chip: keys read once, moved key rows
        # written from registers, moved value rows read and written
        step_bytes = (tokens * row + q_bytes + tokens * 4 + units * spec.budget * 4
                      + moved_rows * row + moved_rows * row * 2)
        if args.shared or not fused_launch(spec, lens0[trig]):
            raise SystemExit(f"{spec.name}: rkv_step runs the three kernels here; "
                             "time it with --three-calls")
        kern = {"step": {"us": region_us, "bytes": step_bytes}}
    total_us = sum(k["us"] for k in kern.values())
    if not (all(k["us"] > 0 for k in kern.values()) and total_us <= ms * 1e3 * 1.05):
        raise RuntimeError(f"implausible event timings {kern} vs {ms} ms per step")
    for k in kern.values():
        k["GB/s"] = round(k["bytes"] / (k["us"] * 1e-6) / 1e9, 1)
        k["us"] = round(k["us"], 2)
    dom = max(kern, key=lambda k: kern[k]["us"])
    achieved = kern[dom]["GB/s"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom}
    tb = measured_traffic(dom, spec.name)
    if tb is not None:
        roofline["traffic"] = tb
    # (not in counter runs: the calibration copy must be the last copy they see)
    peaks = None if args.copy_probe else measured_peaks(torch, stream)
    if peaks:   # the copy rate of our own streaming kernel: the step both reads and writes
        roofline["peak_measured"] = peaks["hbm_stream_copy_GBps"]
        roofline["peak_measured_kind"] = "this repository's streaming copy kernel, 2 GiB buffers"
        roofline["frac_measured"] = round(achieved / peaks["hbm_stream_copy_GBps"], 4)
    extras = {}
    if not (args.no_extras or args.copy_probe or args.three_calls or args.device_lens
            or args.shared or restore):
        extras["roofline_mfma"] = gram_record(spec, case, stream, peaks)
        extras["three_calls"] = three_call_record(spec, case, step, copies, caches, stream)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(spec, case, args.cpu_seconds)

    steps_per_s = 1e3 / ms
    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs, "num_layers": spec.num_layers,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "seq_lens": sorted(set(int(x) for x in lens0)),
                   "budget": spec.budget, "buffer": spec.buffer, "window": spec.window,
                   "mix_lambda": spec.mix_lambda, "layout": spec.layout,
                   "triggered_units": units},
        "tokens_scored_per_s": round(tokens / (ms * 1e-3), 1),
        # sequence tokens whose caches were compressed (sum of the triggered lengths) per second
        "cache_tokens_per_s": round(int(sum(int(n) for n in lens0[trig])) / (ms * 1e-3), 1),
        "entry": ("rkv_score+rkv_select+rkv_compact" if args.three_calls else
                  "rkv_step_device" if args.device_lens else "rkv_step"),
        "selection": "head-shared" if args.shared else "per kv head",
        "roofline": roofline,
        "kernels": kern,
        "kernel_timing": ("HIP events around each kernel" if args.three_calls else
                          "HIP events around the timed region / steps (the table kernel and the step "
                          "kernel per step)" if args.device_lens else
                          "HIP events around the timed region / steps (one kernel per step)")
                         + ("; cache blocks restored between steps outside the timed intervals, "
                            "ms_per_step = mean per-step event interval" if restore else ""),
        "moved_rows": moved_rows,
        "measured_peaks": peaks,
        **extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def gram_record(spec, case, stream, peaks, launches=50):
    """The redundancy through the explicit cosine Gram (rkv_redundancy_gram) on
    the same batch, against the dense bf16 matrix-core peak: 2 N^2 d flops per
    unit (every product of the unit's full N x N Gram, no symmetry used) over
    the kernel's mean launch time (HIP events around back-to-back launches;
    the call only reads the cache)."""
    import numpy as np
    import torch

    from gpu_harness import config_of
    from kv_cache_compression_decode_amd import binding as B

    lens0 = case.lens0.astype(np.int32)
    maxn = int(lens0.max())
    trig = lens0 >= spec.budget + spec.buffer
    red = torch.empty((spec.num_layers * spec.num_seqs * spec.num_kv_heads, maxn),
                      dtype=torch.float32, device="cuda")
    cfg = config_of(spec)
    for _ in range(3):
        B.rkv_redundancy_gram(cfg, case.cache, spec.num_seqs, lens0, red, maxn, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(launches):
        B.rkv_redundancy_gram(cfg, case.cache, spec.num_seqs, lens0, red, maxn, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / launches
    flops = sum(2.0 * int(n) ** 2 * spec.head_dim for n in lens0[trig]) * spec.num_layers * spec.num_kv_heads
    tflops = flops / (us * 1e-6) / 1e12
    rec = {"bound": "mfma", "kernel": "gram", "entry": "rkv_redundancy_gram",
           "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "us": round(us, 2),
           "flops_per_launch": flops,
           "work": "2 N^2 d flops per unit: every product of the full N x N Gram (no symmetry)",
           "traffic": measured_traffic("gram", spec.name), "launches": launches}
    if peaks:
        rec["peak_measured"] = peaks["bf16_gemm_TFLOPs"]
        rec["frac_measured"] = round(tflops / peaks["bf16_gemm_TFLOPs"], 4)
    return rec


def three_call_record(spec, case, step, copies, caches, stream, reps=10):
    """The step as three calls (rkv_score, rkv_select, rkv_compact) on the same
    batch, against 8 TB/s.  Each call is launched reps times back to back
    between one pair of HIP events on its stream (so nothing runs between the
    launches and interval / reps is the call's duration): scoring and
    selection on one cache (they only read it), compaction on reps pristine
    copies prepared beforehand (one more, before the timed launches, takes
    the first launch, which also loads the kernel).  Algorithmic bytes: scoring reads the keys
    once (N d 2 B), the window queries, and writes the scores; selection reads
    the scores and writes the keep lists; compaction reads and writes the
    moved K and V rows and reads the keep lists (once per K and per V
    workgroup)."""
    import numpy as np
    import torch

    lens0 = case.lens0.astype(np.int32)
    trig = lens0 >= spec.budget + spec.buffer
    units = int(trig.sum()) * spec.num_layers * spec.num_kv_heads
    esz = 2 if spec.dtype == "bf16" else 4
    row = spec.head_dim * esz
    tokens = int(sum(int(n) for n in lens0[trig])) * spec.num_layers * spec.num_kv_heads
    reps = min(reps, len(caches) - 1)
    for (kc, vc) in copies[:reps + 1]:
        kc.copy_(case.k)
        vc.copy_(case.v)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    calls = {
        "score": lambda i: step.score(caches[0], case.q, lens0.copy(), stream),
        "select": lambda i: step.select(lens0.copy(), stream),
        "compact": lambda i: step.compact(caches[i + 1], lens0.copy(), stream),
    }
    for name in ("score", "select"):   # warm-up: the first launch of a kernel loads it
        calls[name](0)
    step.compact(caches[0], lens0.copy(), stream)   # copy 0 is the compaction's warm-up
    copies[0][0].copy_(case.k)                      # and is the scoring's input again
    copies[0][1].copy_(case.v)
    torch.cuda.synchronize()
    for j, name in enumerate(("score", "select", "compact")):
        ev[2 * j].record(stream)
        for i in range(reps):
            calls[name](i)
        ev[2 * j + 1].record(stream)
    torch.cuda.synchronize()
    keep = step.keep.view(spec.num_layers, spec.num_seqs, spec.num_kv_heads, spec.budget)
    keep = keep.cpu().numpy()[:, trig].reshape(-1, spec.budget)
    moved = int((keep != np.arange(spec.budget)[None, :]).sum())
    gw = spec.group * spec.window
    nbytes = {"score": tokens * row + units * gw * row + tokens * 4,
              "select": tokens * 4 + units * spec.budget * 4,
              "compact": moved * row * 2 * 2 + units * spec.budget * 4 * 2}
    kern = {}
    for j, name in enumerate(("score", "select", "compact")):
        us = ev[2 * j].elapsed_time(ev[2 * j + 1]) * 1e3 / reps
        gbs = nbytes[name] / (us * 1e-6) / 1e9
        kern[name] = {"us": round(us, 2), "bytes": nbytes[name], "GB/s": round(gbs, 1),
                      "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "bound": "hbm" if name != "select" else "latency",
                      "traffic": measured_traffic(name, spec.name)}
    return {"entry": "rkv_score+rkv_select+rkv_compact", "reps": reps,
            "ms_per_step": round(sum(k["us"] for k in kern.values()) / 1e3, 4),
            "moved_rows": moved, "kernels": kern,
            "kernel_timing": "per call, HIP events around reps back-to-back launches / reps"}


def window_store_bench(args, spec):
    """rkv_window_store for one decode step of the workload's batch: every
    layer's queries (num_seqs x num_q_heads rows of head_dim) into the ring,
    one call.  Algorithmic bytes: the rows read once and written once."""
    import numpy as np
    import torch

    from gpu_harness import config_of
    from kv_cache_compression_decode_amd import binding as B

    steps = 100 if args.steps is None else args.steps
    cfg = config_of(spec)
    dt = torch.int16 if spec.dtype == "bf16" else torch.float32
    L, S, H, d, w = spec.num_layers, spec.num_seqs, spec.num_q_heads, spec.head_dim, spec.window
    q = torch.randn((L, S, H, d), device="cuda").to(dt) if dt == torch.float32 else \
        torch.randint(-2000, 2000, (L, S, H, d), dtype=dt, device="cuda")
    ring = torch.zeros((L, S, H, w, d), dtype=dt, device="cuda")
    ctr = torch.arange(S, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        B.rkv_window_store(cfg, 0, L, q, S, ctr, ring, stream)

    for _ in range(args.warmup):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(steps):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    nbytes = 2 * q.numel() * q.element_size()
    gbs = nbytes / (us * 1e-6) / 1e9
    out = {
        "metric": "window-query ring stores/sec (one decode step's queries, all layers)",
        "value": round(1e6 / us, 2), "unit": "stores/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round((t1 - t0) * 1e3 / steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "num_layers": L, "num_seqs": S, "num_q_heads": H,
                   "head_dim": d, "window": w},
        "entry": "rkv_window_store",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "window_store",
                     "bytes_per_launch": nbytes},
        "kernels": {"window_store": {"us": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1)}},
        "kernel_timing": "HIP events around the timed region / launches (one kernel per launch)",
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def gram_bench(args, spec, case):
    """rkv_redundancy_gram over the workload's triggered units: every unit's
    N x N cosine matrix on the matrix cores, reduced to its row means.  It
    reads the cache only, so all launches use the same cache; one event pair
    around the back-to-back launches gives the launch duration.  Algorithmic
    work: 2 N^2 d flops per unit (every product of the unit's N x N x d Gram)."""
    import numpy as np
    import torch

    from gpu_harness import config_of
    from kv_cache_compression_decode_amd import binding as B

    if spec.dtype != "bf16":
        raise SystemExit(f"{spec.name}: the Gram path takes bf16 caches")
    steps = 100 if args.steps is None else args.steps
    cfg = config_of(spec)
    lens0 = case.lens0.astype(np.int32)
    maxn = int(lens0.max())
    trig = lens0 >= spec.budget + spec.buffer
    units = int(trig.sum()) * spec.num_layers * spec.num_kv_heads
    red = torch.empty((spec.num_layers * spec.num_seqs * spec.num_kv_heads, maxn),
                      dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run():
        B.rkv_redundancy_gram(cfg, case.cache, spec.num_seqs, lens0, red, maxn, stream)

    for _ in range(args.warmup):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(steps):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    ms = (t1 - t0) * 1e3 / steps
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    flops = sum(2.0 * int(n) ** 2 * spec.head_dim for n in lens0[trig]) * spec.num_layers * spec.num_kv_heads
    tflops = flops / (us * 1e-6) / 1e12
    peaks = None if args.copy_probe else measured_peaks(torch, stream)
    out = {
        "metric": "Gram redundancy passes/sec (every triggered unit's N x N cosine matrix); % MFMA roofline",
        "value": round(1e6 / us, 2),
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs, "num_layers": spec.num_layers,
                   "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
                   "seq_lens": sorted(set(int(x) for x in lens0)), "layout": spec.layout,
                   "triggered_units": units},
        "entry": "rkv_redundancy_gram",
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("gram", spec.name), "kernel": "gram",
                     "flops_per_launch": flops,
                     **({"peak_measured": peaks["bf16_gemm_TFLOPs"],
                         "frac_measured": round(tflops / peaks["bf16_gemm_TFLOPs"], 4)} if peaks else {})},
        "measured_peaks": peaks,
        "kernels": {"gram": {"us": round(us, 2)}},
        "kernel_timing": "HIP events around the timed region / steps (one kernel per launch)",
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def kara_bench(args, spec, case, window_len=128, keep=32, anchors=4, radius=2):
    """rkv_kara_step on the workload's caches: every sequence's last window_len
    tokens are its uncompressed tail, scored by bidirectional attention of
    their own queries and cut to `keep`.  Compaction is in place, so each step
    gets a pristine cache copy prepared before the timed region; one event
    pair around the back-to-back launches.  Algorithmic bytes per unit: the
    window tokens' queries (G W d 2) and keys (W d 2) read once, scores
    (W 4) and keep list (keep 4) written; per moved row, its K row written
    (the keys were read for the scores) and its V row read and written."""
    import numpy as np
    import torch

    import rkv_synth as syn
    from gpu_harness import config_of, to_dev
    from kv_cache_compression_decode_amd import binding as B

    if spec.dtype != "bf16" or spec.layout != "contiguous":
        raise SystemExit(f"{spec.name}: --kara times bf16 contiguous workloads")
    steps = 50 if args.steps is None else args.steps
    nsteps = args.warmup + steps
    cfg = config_of(spec)
    kc = B.rkv_kara_config(window_len, keep, anchors, radius)
    lens0 = case.lens0.astype(np.int32)
    tails0 = lens0 - window_len
    q = to_dev(syn.build_queries(spec.with_(window=window_len)))
    units = spec.num_seqs * spec.num_layers * spec.num_kv_heads
    scores = torch.empty(units * window_len, dtype=torch.float32, device="cuda")
    keep_t = torch.empty(units * keep, dtype=torch.int32, device="cuda")
    copies = [(case.k.clone(), case.v.clone()) for _ in range(nsteps)]
    caches = [B.make_cache(kk, vv, capacity=case.cap) for kk, vv in copies]
    stream = torch.cuda.current_stream()

    def run(i):
        B.rkv_kara_step(cfg, kc, caches[i], q, spec.num_seqs, lens0.copy(), tails0.copy(), scores,
                        keep_t, None, 0, None, None, 0, stream)

    for i in range(args.warmup):
        run(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.warmup, nsteps):
        run(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / steps
    kept = keep_t.view(units, keep).cpu().numpy()
    first = (lens0 - window_len)[0]
    moved = int((kept != first + np.arange(keep)[None, :]).sum())
    row = spec.head_dim * 2
    # the window keys are read once (for the scores); a moved row's K is
    # written, its V read and written
    nbytes = (units * (spec.group * window_len * row + window_len * row + window_len * 4 + keep * 4)
              + moved * row * 3)
    gbs = nbytes / (us * 1e-6) / 1e9
    out = {
        "metric": "KARA-style window steps/sec (score, Token2Chunk-select and compact every unit's window)",
        "value": round(1e6 / us, 2), "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round((t1 - t0) * 1e3 / steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs, "num_layers": spec.num_layers,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "seq_lens": sorted(set(int(x) for x in lens0)),
                   "window_len": window_len, "keep": keep, "anchors": anchors, "radius": radius,
                   "units": units},
        "entry": "rkv_kara_step",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("kara", spec.name),
                     "kernel": "kara", "bytes_per_launch": nbytes},
        "kernels": {"kara": {"us": round(us, 2), "bytes": nbytes, "GB/s": round(gbs, 1)}},
        "moved_rows": moved,
        "kernel_timing": "HIP events around the timed region / steps (one kernel per step)",
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
