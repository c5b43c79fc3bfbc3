"""Build librkv.so (the HIP kernels and the C ABI of include/rkv.h) for gfx950.

Usage: python -m kv_cache_compression_decode_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "librkv.so")
# streaming bandwidth kernels the benchmark measures HBM with (not part of the step)
MEMBENCH_SRC = os.path.join(PKG, "membench", "rkv_membench.hip")
MEMBENCH_OUT = os.path.join(PKG, "librkv_membench.so")
EXAMPLE = os.path.join(PKG, "rkv_c_example")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["rkv_api.hip", "rkv_score.hip", "rkv_select.hip", "rkv_compact.hip", "rkv_table.hip",
           "rkv_gram.hip", "rkv_window.hip", "rkv_kara.hip"] + [
    f"rkv_score_{dt}_d{d}_{lay}.hip" for dt in ("bf16", "f32") for d in (64, 128)
    for lay in ("contig", "paged")]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# per-source additions: the Gram and KARA kernels use every matrix-core
# result on the vector ALUs (column scaling; the window softmax), so their
# MFMAs write ordinary VGPRs (no copy out of AGPRs)
EXTRA_FLAGS = {"rkv_gram.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "rkv_kara.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = OUT + ".tmp"
    # --no-undefined: a kernel the compiler dropped shows up here, not at load time
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined",
          "-Wl,-soname,librkv.so", *objs, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    tmp = MEMBENCH_OUT + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", "-Wl,--no-undefined", "-Wl,-soname,librkv_membench.so",
          MEMBENCH_SRC, "-o", tmp], verbose)
    os.replace(tmp, MEMBENCH_OUT)
    # a caller of the C ABI without Python (run by the GPU tests), linked against
    # the library next to it
    _run([HIPCC, *FLAGS, os.path.join(PKG, "examples", "rkv_c_example.cpp"), f"-L{PKG}", "-lrkv",
          "-Wl,-rpath,$ORIGIN", "-o", EXAMPLE], verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
