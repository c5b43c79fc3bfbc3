"""Seeded synthetic inputs for the R-KV decode-time compression step.

This module is the only code shared by the CPU oracle side (tests, the CPU
baseline) and the HIP side (tests, bench).  It draws random numbers, shapes
them and encodes them to the storage dtype; it holds none of the method's
arithmetic (no attention, no similarity, no selection, no compaction).

Workload shapes follow the pages' settings: a 7-8B reasoning model decoding
with kv_budget 1024, window_size 8, mix_lambda 0.1 and divide_length 128
(R-KV project page on hysenlabs.com, section "Installing R-KV and running a
first math evaluation"), block sizes of 16 for a paged pool (hotdry blog post
on R-KV / EvolKV / Ada-KV, section on Ada-KV).

Draw order (every stream is ``numpy.random.default_rng([seed, tag, ...])``,
so any (sequence, layer) chunk can be regenerated on its own):

  tag 0, [seed, 0]          sequence lengths (only for ranged lengths)
  tag 1, [seed, 1, s]       per-sequence duplicate fraction (ranged only),
                            then the duplicate plan of sequence s
  tag 2, [seed, 2, l]       per-(layer, kv-head) key mean, N(0, key_mean_std)
  tag 3, [seed, 3, s, l]    keys: base N(mu, 1) for (Hkv, N, d), then the
                            near-duplicate noise N(0, dup_noise_std) for
                            (duplicated tokens, Hkv, d) in plan order
  tag 4, [seed, 4, s, l]    values N(0, 1), (Hkv, N, d)
  tag 5, [seed, 5, s, l]    window queries N(0, 1), (Hq, window, d)
  tag 6, [seed, 6]          permutation of the paged pool's block ids

Normal draws are float32; bf16 storage rounds them to nearest-even.
``N(a, b)`` in the workload descriptions is read as (mean, standard deviation).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Spec", "CONFIGS", "config", "seq_lens",
    "dup_plan", "key_means", "keys", "values", "queries", "block_table",
    "to_bf16_bits", "storage_dtype", "build_contiguous", "build_paged",
    "build_queries", "CANARY_BF16", "CANARY_F32",
]

# Bit pattern written into cache rows that hold no token (slots >= N, pool
# blocks nobody references).  Any kernel that writes there is caught.
CANARY_BF16 = np.uint16(0x7F7F)          # a large finite bf16 value
CANARY_F32 = np.float32(-12345.678)


@dataclass(frozen=True)
class Spec:
    """One synthetic workload: shapes, lengths, distribution and seed."""
    name: str
    seed: int
    num_seqs: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    budget: int
    buffer: int
    window: int
    mix_lambda: float
    layout: str = "contiguous"      # "contiguous" or "paged"
    block_size: int = 16
    num_blocks: int = 0             # paged: blocks per layer in the pool
    # lengths: either fixed per sequence or uniform integers in [lo, hi]
    lens: Optional[Tuple[int, ...]] = None
    len_range: Optional[Tuple[int, int]] = None
    key_mean_std: float = 0.0       # 0 -> keys N(0, 1)
    dup_mode: str = "scatter"       # "scatter" single tokens, or "runs"
    dup_frac: float = 0.0           # fixed fraction of duplicated tokens
    dup_frac_range: Optional[Tuple[float, float]] = None
    dup_run_range: Tuple[int, int] = (16, 64)
    dup_noise_std: float = 0.01

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


def _cfg(**kw) -> Spec:
    return Spec(**kw)


# The five workloads.  Index i uses seed i.
CONFIGS: Tuple[Spec, ...] = (
    # 0: tiny fp32 step, one unit
    _cfg(name="tiny-f32", seed=0, num_seqs=1, num_layers=1, num_q_heads=4,
         num_kv_heads=1, head_dim=64, dtype="f32", budget=128, buffer=32,
         window=8, mix_lambda=0.1, lens=(160,), key_mean_std=0.0,
         dup_mode="scatter", dup_frac=0.20),
    # 1: Llama-8B-shaped single sequence, 32 layers in one launch
    _cfg(name="llama8b-1seq", seed=1, num_seqs=1, num_layers=32, num_q_heads=32,
         num_kv_heads=8, head_dim=128, dtype="bf16", budget=1024, buffer=128,
         window=8, mix_lambda=0.1, lens=(1152,), key_mean_std=0.5,
         dup_mode="scatter", dup_frac=0.30),
    # 2: Qwen-7B-shaped ragged batch; only lengths >= B + buffer trigger
    _cfg(name="qwen7b-ragged16", seed=2, num_seqs=16, num_layers=28, num_q_heads=28,
         num_kv_heads=4, head_dim=128, dtype="bf16", budget=2048, buffer=128,
         window=8, mix_lambda=0.1, len_range=(2049, 2176), key_mean_std=0.5,
         dup_mode="scatter", dup_frac_range=(0.1, 0.5)),
    # 3: paged Llama-8B shape, 8 sequences at the trigger point
    _cfg(name="llama8b-paged8", seed=3, num_seqs=8, num_layers=32, num_q_heads=32,
         num_kv_heads=8, head_dim=128, dtype="bf16", budget=4096, buffer=256,
         window=8, mix_lambda=0.1, layout="paged", block_size=16, num_blocks=65536,
         lens=(4352,) * 8, key_mean_std=0.5, dup_mode="scatter", dup_frac=0.30),
    # 4: 70B-shaped batch of 32 sequences, duplicate runs
    _cfg(name="70b-batch32", seed=4, num_seqs=32, num_layers=80, num_q_heads=64,
         num_kv_heads=8, head_dim=128, dtype="bf16", budget=1024, buffer=128,
         window=8, mix_lambda=0.1, lens=(1152,) * 32, key_mean_std=0.5,
         dup_mode="runs", dup_frac=0.40),
)


def config(i: int) -> Spec:
    return CONFIGS[i]


def storage_dtype(spec: Spec):
    return np.uint16 if spec.dtype == "bf16" else np.float32


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Inputs are finite by construction (normal draws), so no NaN handling.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = b + np.uint32(0x7FFF)
    r += lsb
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _encode(spec: Spec, x: np.ndarray) -> np.ndarray:
    return to_bf16_bits(x) if spec.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


# ---------------------------------------------------------------- lengths

def seq_lens(spec: Spec) -> np.ndarray:
    if spec.lens is not None:
        assert len(spec.lens) == spec.num_seqs
        return np.asarray(spec.lens, dtype=np.int32)
    lo, hi = spec.len_range
    rng = np.random.default_rng([spec.seed, 0])
    return rng.integers(lo, hi + 1, size=spec.num_seqs).astype(np.int32)


# ---------------------------------------------------------------- duplicates

def dup_plan(spec: Spec, s: int, n: int) -> list:
    """Near-duplicate plan of sequence s with n cached tokens.

    Returns ascending (dst, src, length) spans, src + length <= dst.  The same
    plan applies to every layer and kv-head of the sequence; each duplicated
    element gets fresh noise.
    """
    rng = np.random.default_rng([spec.seed, 1, s])
    frac = spec.dup_frac
    if spec.dup_frac_range is not None:
        lo, hi = spec.dup_frac_range
        frac = float(rng.uniform(lo, hi))
    if frac <= 0.0 or n < 2:
        return []
    if spec.dup_mode == "scatter":
        count = int(math.floor(frac * n))
        count = min(count, n - 1)
        dst = np.sort(rng.choice(np.arange(1, n), size=count, replace=False))
        src = [int(rng.integers(0, int(d))) for d in dst]
        return [(int(d), int(c), 1) for d, c in zip(dst, src)]
    if spec.dup_mode == "runs":
        rlo, rhi = spec.dup_run_range
        target = frac * n
        covered = 0
        taken = np.zeros(n, dtype=bool)
        runs = []
        attempts = 0
        while covered < target and attempts < 100000:
            attempts += 1
            length = int(rng.integers(rlo, rhi + 1))
            if 2 * length > n:
                continue
            dst = int(rng.integers(length, n - length + 1))
            if taken[dst:dst + length].any():
                continue
            taken[dst:dst + length] = True
            covered += length
            runs.append((dst, length))
        runs.sort()
        out = []
        for dst, length in runs:
            src = int(rng.integers(0, dst - length + 1))
            out.append((dst, src, length))
        return out
    raise ValueError(spec.dup_mode)


# ---------------------------------------------------------------- tensors

def key_means(spec: Spec, layer: int) -> np.ndarray:
    if spec.key_mean_std == 0.0:
        return np.zeros((spec.num_kv_heads, spec.head_dim), np.float32)
    rng = np.random.default_rng([spec.seed, 2, layer])
    return (rng.standard_normal((spec.num_kv_heads, spec.head_dim), dtype=np.float32)
            * np.float32(spec.key_mean_std))


def _keys_f32(spec: Spec, s: int, l: int, n: int, plan=None) -> np.ndarray:
    rng = np.random.default_rng([spec.seed, 3, s, l])
    hk, d = spec.num_kv_heads, spec.head_dim
    k = rng.standard_normal((hk, n, d), dtype=np.float32)
    k += key_means(spec, l)[:, None, :]
    plan = dup_plan(spec, s, n) if plan is None else plan
    total = sum(length for _, _, length in plan)
    if total:
        noise = rng.standard_normal((total, hk, d), dtype=np.float32)
        noise *= np.float32(spec.dup_noise_std)
        o = 0
        for dst, src, length in plan:
            k[:, dst:dst + length, :] = (k[:, src:src + length, :]
                                         + noise[o:o + length].transpose(1, 0, 2))
            o += length
    return k


def keys(spec: Spec, s: int, l: int, n: Optional[int] = None, plan=None) -> np.ndarray:
    """Keys of (sequence s, layer l): (Hkv, N, d) in storage dtype."""
    n = int(seq_lens(spec)[s]) if n is None else n
    return _encode(spec, _keys_f32(spec, s, l, n, plan))


def values(spec: Spec, s: int, l: int, n: Optional[int] = None) -> np.ndarray:
    n = int(seq_lens(spec)[s]) if n is None else n
    rng = np.random.default_rng([spec.seed, 4, s, l])
    return _encode(spec, rng.standard_normal((spec.num_kv_heads, n, spec.head_dim),
                                             dtype=np.float32))


def queries(spec: Spec, s: int, l: int) -> np.ndarray:
    """Window queries of (sequence s, layer l): (Hq, window, d) in storage dtype."""
    rng = np.random.default_rng([spec.seed, 5, s, l])
    return _encode(spec, rng.standard_normal((spec.num_q_heads, spec.window, spec.head_dim),
                                             dtype=np.float32))


def blocks_per_seq(spec: Spec, lens: Optional[np.ndarray] = None) -> int:
    lens = seq_lens(spec) if lens is None else lens
    return int(-(-int(lens.max()) // spec.block_size))


def block_table(spec: Spec) -> np.ndarray:
    """(S, max_blocks) int32 physical block ids: a seeded permutation of the
    pool, first S * max_blocks entries, row-major.  Shared by all layers."""
    mb = blocks_per_seq(spec)
    need = spec.num_seqs * mb
    assert need <= spec.num_blocks, "pool too small"
    rng = np.random.default_rng([spec.seed, 6])
    perm = rng.permutation(spec.num_blocks)[:need]
    return perm.reshape(spec.num_seqs, mb).astype(np.int32)


# ---------------------------------------------------------------- full arrays

def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _canary(spec: Spec):
    return CANARY_BF16 if spec.dtype == "bf16" else CANARY_F32


def build_queries(spec: Spec) -> np.ndarray:
    """(L, S, Hq, window, d) window queries."""
    out = np.empty((spec.num_layers, spec.num_seqs, spec.num_q_heads, spec.window,
                    spec.head_dim), storage_dtype(spec))
    for l in range(spec.num_layers):
        for s in range(spec.num_seqs):
            out[l, s] = queries(spec, s, l)
    return out


def build_contiguous(spec: Spec, capacity: Optional[int] = None, out_k=None, out_v=None):
    """K, V as (L, S, Hkv, capacity, d); slots >= N hold the canary."""
    lens = seq_lens(spec)
    cap = int(lens.max()) if capacity is None else capacity
    shape = (spec.num_layers, spec.num_seqs, spec.num_kv_heads, cap, spec.head_dim)
    k = np.empty(shape, storage_dtype(spec)) if out_k is None else out_k
    v = np.empty(shape, storage_dtype(spec)) if out_v is None else out_v
    plans = [dup_plan(spec, s, int(lens[s])) for s in range(spec.num_seqs)]

    def job(idx):
        l, s = divmod(idx, spec.num_seqs)
        n = int(lens[s])
        k[l, s, :, :n] = keys(spec, s, l, n, plans[s])
        v[l, s, :, :n] = values(spec, s, l, n)
        k[l, s, :, n:] = _canary(spec)
        v[l, s, :, n:] = _canary(spec)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(spec.num_layers * spec.num_seqs)))
    return k, v


def scatter_paged(spec: Spec, pool: np.ndarray, chunk: np.ndarray, l: int, bt_row: np.ndarray):
    """Write one (Hkv, N, d) chunk of layer l into pool (L, nblk, Hkv, bs, d)."""
    bs = spec.block_size
    n = chunk.shape[1]
    for b in range(-(-n // bs)):
        rows = chunk[:, b * bs:(b + 1) * bs, :]
        pool[l, bt_row[b], :, :rows.shape[1], :] = rows


def build_paged(spec: Spec, out_k=None, out_v=None, fill_pool: bool = True):
    """Paged pools (L, num_blocks, Hkv, bs, d) + block table.

    Unreferenced blocks and the tail of a partial last block hold the canary.
    With ``fill_pool=False`` only referenced blocks are written (callers that
    canary-fill on their own, e.g. directly on the device).
    """
    lens = seq_lens(spec)
    bt = block_table(spec)
    shape = (spec.num_layers, spec.num_blocks, spec.num_kv_heads, spec.block_size,
             spec.head_dim)
    k = np.empty(shape, storage_dtype(spec)) if out_k is None else out_k
    v = np.empty(shape, storage_dtype(spec)) if out_v is None else out_v
    if fill_pool:
        k[...] = _canary(spec)
        v[...] = _canary(spec)
    plans = [dup_plan(spec, s, int(lens[s])) for s in range(spec.num_seqs)]

    def job(idx):
        l, s = divmod(idx, spec.num_seqs)
        n = int(lens[s])
        scatter_paged(spec, k, keys(spec, s, l, n, plans[s]), l, bt[s])
        scatter_paged(spec, v, values(spec, s, l, n), l, bt[s])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range(spec.num_layers * spec.num_seqs)))
    return k, v, bt
