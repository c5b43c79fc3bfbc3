"""ctypes binding of librkv.so (the C ABI in include/rkv.h).

Argument marshalling only: every function forwards to the C entry point of
the same name; device buffers may be given as torch tensors, raw integer
addresses or None (NULL).  Nothing here computes any part of the step, and
there is no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p
from typing import Optional

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librkv.so")

RKV_OK = 0
RKV_ERR_INVALID_ARG = 1
RKV_ERR_UNSUPPORTED = 2
RKV_ERR_WORKSPACE = 3
RKV_ERR_HIP = 4
RKV_ERR_DEVICE_CHECK = 5

RKV_DEVICE_SPAN_TIMEOUT = 1
RKV_DEVICE_BAD_BLOCK_ID = 2

RKV_DTYPE_F32 = 0
RKV_DTYPE_BF16 = 1
RKV_LAYOUT_CONTIGUOUS = 0
RKV_LAYOUT_PAGED = 1

RKV_MAX_LEN = 32768
RKV_MAX_WINDOW_ROWS = 142

# Every function declared in include/rkv.h.
EXPORTS = ("rkv_status_string", "rkv_last_error", "rkv_is_triggered", "rkv_workspace_size",
           "rkv_redundancy_gram", "rkv_window_store",
           "rkv_score", "rkv_select", "rkv_compact", "rkv_step",
           "rkv_step_device_workspace_size", "rkv_step_device", "rkv_device_status",
           "rkv_set_span_wait_us", "rkv_step_noalloc", "rkv_kara_step")


class rkv_config(ctypes.Structure):
    _fields_ = [("num_layers", c_int32), ("num_q_heads", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("budget", c_int32), ("buffer", c_int32),
                ("window", c_int32), ("mix_lambda", c_float), ("dtype", c_int32),
                ("layout", c_int32), ("block_size", c_int32), ("shared_selection", c_int32),
                ("check_block_table", c_int32)]


class rkv_cache(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("layer_stride", ctypes.c_int64),
                ("capacity", c_int32),
                ("num_blocks", c_int32), ("block_table", c_void_p),
                ("max_blocks_per_seq", c_int32)]


class rkv_kara_config(ctypes.Structure):
    _fields_ = [("window_len", c_int32), ("keep", c_int32), ("anchors", c_int32),
                ("radius", c_int32)]


class RkvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librkv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m kv_cache_compression_decode_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = POINTER
    lib.rkv_status_string.argtypes = [c_int32]
    lib.rkv_status_string.restype = ctypes.c_char_p
    lib.rkv_last_error.argtypes = []
    lib.rkv_last_error.restype = ctypes.c_char_p
    lib.rkv_is_triggered.argtypes = [P(rkv_config), c_int32]
    lib.rkv_is_triggered.restype = c_int32
    lib.rkv_workspace_size.argtypes = [P(rkv_config), c_int32, c_int32]
    lib.rkv_workspace_size.restype = c_size_t
    lib.rkv_score.argtypes = [P(rkv_config), P(rkv_cache), c_void_p, c_int32, P(c_int32),
                              c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.rkv_score.restype = c_int32
    lib.rkv_redundancy_gram.argtypes = [P(rkv_config), P(rkv_cache), c_int32, P(c_int32),
                                        c_void_p, c_int32, c_void_p]
    lib.rkv_redundancy_gram.restype = c_int32
    lib.rkv_window_store.argtypes = [P(rkv_config), c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                     c_void_p, c_void_p]
    lib.rkv_window_store.restype = c_int32
    lib.rkv_select.argtypes = [P(rkv_config), c_int32, P(c_int32), c_void_p, c_int32, c_void_p,
                               c_void_p, c_size_t, c_void_p]
    lib.rkv_select.restype = c_int32
    lib.rkv_compact.argtypes = [P(rkv_config), P(rkv_cache), c_int32, P(c_int32), c_void_p,
                                c_void_p, c_int32, P(c_int32), c_void_p, c_size_t, c_void_p]
    lib.rkv_compact.restype = c_int32
    lib.rkv_step.argtypes = [P(rkv_config), P(rkv_cache), c_void_p, c_int32, P(c_int32), c_void_p,
                             c_int32, c_void_p, c_void_p, c_int32, P(c_int32), c_void_p, c_size_t,
                             c_void_p]
    lib.rkv_step.restype = c_int32
    lib.rkv_step_device_workspace_size.argtypes = [P(rkv_config), c_int32, c_int32]
    lib.rkv_step_device_workspace_size.restype = c_size_t
    lib.rkv_step_device.argtypes = [P(rkv_config), P(rkv_cache), c_void_p, c_int32, c_void_p,
                                    c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                    c_void_p, c_void_p, c_size_t, c_void_p]
    lib.rkv_step_device.restype = c_int32
    lib.rkv_step_noalloc.argtypes = [P(rkv_config), P(rkv_cache), c_void_p, c_int32, P(c_int32),
                                     c_void_p, c_int32, c_void_p, c_void_p, c_int32, P(c_int32),
                                     c_void_p]
    lib.rkv_step_noalloc.restype = c_int32
    lib.rkv_kara_step.argtypes = [P(rkv_config), P(rkv_kara_config), P(rkv_cache), c_void_p, c_int32,
                                  P(c_int32), P(c_int32), c_void_p, c_void_p, c_void_p, c_int32,
                                  P(c_int32), c_void_p, c_size_t, c_void_p]
    lib.rkv_kara_step.restype = c_int32
    lib.rkv_device_status.argtypes = [c_void_p, c_void_p, P(ctypes.c_uint32)]
    lib.rkv_device_status.restype = c_int32
    lib.rkv_set_span_wait_us.argtypes = [ctypes.c_int64]
    lib.rkv_set_span_wait_us.restype = ctypes.c_int64
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().rkv_status_string(status).decode()
    except Exception:  # noqa: BLE001 - name lookup must not hide the real error
        return f"status {status}"


def _ptr(x) -> Optional[int]:
    """Device or host address of a torch tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)!r}")


def _stream(s) -> Optional[int]:
    if s is None or isinstance(s, int):
        return s
    return s.cuda_stream   # torch.cuda.Stream


def _lens(a) -> Optional[np.ndarray]:
    """Host int32 view of sequence lengths; arrays are used in place."""
    if a is None:
        return None
    if isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i32p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(POINTER(c_int32))


def _check(status: int) -> None:
    if status != RKV_OK:
        raise RkvError(status, load().rkv_last_error().decode())


# ------------------------------------------------------------------ entry points

def rkv_status_string(status: int) -> str:
    return load().rkv_status_string(status).decode()


def rkv_last_error() -> str:
    return load().rkv_last_error().decode()


def rkv_is_triggered(cfg: rkv_config, length: int) -> int:
    return load().rkv_is_triggered(ctypes.byref(cfg), length)


def rkv_workspace_size(cfg: rkv_config, num_seqs: int, max_len: int) -> int:
    return load().rkv_workspace_size(ctypes.byref(cfg), num_seqs, max_len)


def rkv_score(cfg, cache, q_window, num_seqs, seq_lens, scores, score_stride,
              importance=None, redundancy=None, workspace=None, workspace_bytes=0,
              stream=None) -> None:
    lens = _lens(seq_lens)
    _check(load().rkv_score(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q_window), num_seqs,
                            _i32p(lens), _ptr(scores), score_stride, _ptr(importance),
                            _ptr(redundancy), _ptr(workspace), workspace_bytes, _stream(stream)))


def rkv_window_store(cfg, layer0, layer_count, q_step, num_seqs, d_steps, q_window,
                     stream=None) -> None:
    """d_steps: device int32 [num_seqs] (torch tensor or address)."""
    _check(load().rkv_window_store(ctypes.byref(cfg), layer0, layer_count, _ptr(q_step), num_seqs,
                                   _ptr(d_steps), _ptr(q_window), _stream(stream)))


def rkv_redundancy_gram(cfg, cache, num_seqs, seq_lens, redundancy, stride, stream=None) -> None:
    lens = _lens(seq_lens)
    _check(load().rkv_redundancy_gram(ctypes.byref(cfg), ctypes.byref(cache), num_seqs,
                                      _i32p(lens), _ptr(redundancy), stride, _stream(stream)))


def rkv_select(cfg, num_seqs, seq_lens, scores, score_stride, keep, workspace=None,
               workspace_bytes=0, stream=None) -> None:
    lens = _lens(seq_lens)
    _check(load().rkv_select(ctypes.byref(cfg), num_seqs, _i32p(lens), _ptr(scores),
                             score_stride, _ptr(keep), _ptr(workspace), workspace_bytes,
                             _stream(stream)))


def rkv_compact(cfg, cache, num_seqs, seq_lens: np.ndarray, keep, free_blocks=None,
                free_capacity=0, free_counts: Optional[np.ndarray] = None, workspace=None,
                workspace_bytes=0, stream=None) -> None:
    """seq_lens must be a C-contiguous int32 numpy array: it is updated in place
    (triggered sequences become `budget` long).  free_counts likewise."""
    if not (isinstance(seq_lens, np.ndarray) and seq_lens.dtype == np.int32
            and seq_lens.flags.c_contiguous):
        raise TypeError("seq_lens must be a C-contiguous int32 numpy array (updated in place)")
    if free_counts is not None and not (free_counts.dtype == np.int32
                                        and free_counts.flags.c_contiguous):
        raise TypeError("free_counts must be a C-contiguous int32 numpy array")
    _check(load().rkv_compact(ctypes.byref(cfg), ctypes.byref(cache), num_seqs, _i32p(seq_lens),
                              _ptr(keep), _ptr(free_blocks), free_capacity, _i32p(free_counts),
                              _ptr(workspace), workspace_bytes, _stream(stream)))


def rkv_step(cfg, cache, q_window, num_seqs, seq_lens: np.ndarray, scores, score_stride, keep,
             free_blocks=None, free_capacity=0, free_counts: Optional[np.ndarray] = None,
             workspace=None, workspace_bytes=0, stream=None) -> None:
    """seq_lens (C-contiguous int32 numpy) is updated in place, as by rkv_compact."""
    if not (isinstance(seq_lens, np.ndarray) and seq_lens.dtype == np.int32
            and seq_lens.flags.c_contiguous):
        raise TypeError("seq_lens must be a C-contiguous int32 numpy array (updated in place)")
    if free_counts is not None and not (free_counts.dtype == np.int32
                                        and free_counts.flags.c_contiguous):
        raise TypeError("free_counts must be a C-contiguous int32 numpy array")
    _check(load().rkv_step(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q_window), num_seqs,
                           _i32p(seq_lens), _ptr(scores), score_stride, _ptr(keep),
                           _ptr(free_blocks), free_capacity, _i32p(free_counts),
                           _ptr(workspace), workspace_bytes, _stream(stream)))


def rkv_step_device_workspace_size(cfg: rkv_config, num_seqs: int, max_len: int) -> int:
    return load().rkv_step_device_workspace_size(ctypes.byref(cfg), num_seqs, max_len)


def rkv_step_device(cfg, cache, q_window, num_seqs, d_seq_lens, max_len, scores, score_stride,
                    keep, free_blocks=None, free_capacity=0, d_free_counts=None, workspace=None,
                    workspace_bytes=0, stream=None) -> None:
    """d_seq_lens and d_free_counts are device int32 buffers (torch tensors or
    addresses); the lengths are updated on the device."""
    _check(load().rkv_step_device(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q_window),
                                  num_seqs, _ptr(d_seq_lens), max_len, _ptr(scores),
                                  score_stride, _ptr(keep), _ptr(free_blocks), free_capacity,
                                  _ptr(d_free_counts), _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


def rkv_step_noalloc(cfg, cache, q_window, num_seqs, seq_lens: np.ndarray, scores, score_stride,
                     keep, free_blocks=None, free_capacity=0,
                     free_counts: Optional[np.ndarray] = None, stream=None) -> None:
    """rkv_step with the library's own scratch instead of a workspace."""
    if not (isinstance(seq_lens, np.ndarray) and seq_lens.dtype == np.int32
            and seq_lens.flags.c_contiguous):
        raise TypeError("seq_lens must be a C-contiguous int32 numpy array (updated in place)")
    if free_counts is not None and not (free_counts.dtype == np.int32
                                        and free_counts.flags.c_contiguous):
        raise TypeError("free_counts must be a C-contiguous int32 numpy array")
    _check(load().rkv_step_noalloc(ctypes.byref(cfg), ctypes.byref(cache), _ptr(q_window),
                                   num_seqs, _i32p(seq_lens), _ptr(scores), score_stride,
                                   _ptr(keep), _ptr(free_blocks), free_capacity,
                                   _i32p(free_counts), _stream(stream)))


def rkv_kara_step(cfg, kc, cache, q_tail, num_seqs, seq_lens: np.ndarray, tail_start: np.ndarray,
                  scores, keep, free_blocks=None, free_capacity=0,
                  free_counts: Optional[np.ndarray] = None, workspace=None, workspace_bytes=0,
                  stream=None) -> None:
    """seq_lens and tail_start (C-contiguous int32 numpy) are updated in place."""
    for name, arr in (("seq_lens", seq_lens), ("tail_start", tail_start)):
        if not (isinstance(arr, np.ndarray) and arr.dtype == np.int32 and arr.flags.c_contiguous):
            raise TypeError(f"{name} must be a C-contiguous int32 numpy array (updated in place)")
    if free_counts is not None and not (free_counts.dtype == np.int32
                                        and free_counts.flags.c_contiguous):
        raise TypeError("free_counts must be a C-contiguous int32 numpy array")
    _check(load().rkv_kara_step(ctypes.byref(cfg), ctypes.byref(kc), ctypes.byref(cache),
                                _ptr(q_tail), num_seqs, _i32p(seq_lens), _i32p(tail_start),
                                _ptr(scores), _ptr(keep), _ptr(free_blocks), free_capacity,
                                _i32p(free_counts), _ptr(workspace), workspace_bytes,
                                _stream(stream)))


def rkv_device_status(workspace, stream=None) -> int:
    """The workspace's status word (waits for the stream): 0, or the
    RKV_DEVICE_* flags of the checks that failed.  workspace None: the
    scratch of rkv_step_noalloc on the current device.  Other errors raise."""
    flags = ctypes.c_uint32(0)
    st = load().rkv_device_status(_ptr(workspace), _stream(stream), ctypes.byref(flags))
    if st not in (RKV_OK, RKV_ERR_DEVICE_CHECK):
        _check(st)
    return int(flags.value)


def rkv_set_span_wait_us(microseconds: int) -> int:
    return int(load().rkv_set_span_wait_us(microseconds))


# ------------------------------------------------------------------ helpers

def make_config(num_layers, num_q_heads, num_kv_heads, head_dim, budget, buffer, window,
                mix_lambda, dtype="bf16", layout="contiguous", block_size=16,
                shared_selection=False, check_block_table=False) -> rkv_config:
    return rkv_config(num_layers, num_q_heads, num_kv_heads, head_dim, budget, buffer, window,
                      mix_lambda, RKV_DTYPE_BF16 if dtype == "bf16" else RKV_DTYPE_F32,
                      RKV_LAYOUT_PAGED if layout == "paged" else RKV_LAYOUT_CONTIGUOUS,
                      block_size, 1 if shared_selection else 0, 1 if check_block_table else 0)


def make_cache(k, v, capacity=0, num_blocks=0, block_table=None, max_blocks_per_seq=0,
               layer_stride=0) -> rkv_cache:
    return rkv_cache(_ptr(k), _ptr(v), layer_stride, capacity, num_blocks, _ptr(block_table),
                     max_blocks_per_seq)
