"""One R-KV compression step over torch device tensors.

Owns the buffers a batch shape needs (workspace, scores, keep list) and calls
the C entry points on one stream: the three steps in order, rkv_step, or
rkv_step_device (lengths on the device).  Argument marshalling only:
the work is done by librkv.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding as B  # noqa: N812


class RKVStep:
    def __init__(self, cfg: B.rkv_config, num_seqs: int, max_len: int, device="cuda",
                 keep_parts: bool = False, free_capacity: int = 0):
        import torch
        self.cfg = cfg
        self.num_seqs = num_seqs
        self.max_len = max_len
        rows = cfg.num_layers * num_seqs * cfg.num_kv_heads
        self.ws_bytes = max(256, B.rkv_workspace_size(cfg, num_seqs, max_len))
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.scores = torch.empty(rows * max_len, dtype=torch.float32, device=device)
        self.importance = torch.empty_like(self.scores) if keep_parts else None
        self.redundancy = torch.empty_like(self.scores) if keep_parts else None
        self.keep = torch.empty(rows * cfg.budget, dtype=torch.int32, device=device)
        self.free_capacity = free_capacity
        self.free_blocks = (torch.empty(max(1, free_capacity), dtype=torch.int32, device=device)
                            if free_capacity else None)
        self.free_counts = np.zeros(num_seqs, dtype=np.int32)

    def score(self, cache: B.rkv_cache, q_window, seq_lens, stream=None) -> None:
        B.rkv_score(self.cfg, cache, q_window, self.num_seqs, seq_lens, self.scores, self.max_len,
                    self.importance, self.redundancy, self.workspace, self.ws_bytes, stream)

    def select(self, seq_lens, stream=None) -> None:
        B.rkv_select(self.cfg, self.num_seqs, seq_lens, self.scores, self.max_len, self.keep,
                     self.workspace, self.ws_bytes, stream)

    def compact(self, cache: B.rkv_cache, seq_lens: np.ndarray, stream=None) -> None:
        B.rkv_compact(self.cfg, cache, self.num_seqs, seq_lens, self.keep, self.free_blocks,
                      self.free_capacity, self.free_counts, self.workspace, self.ws_bytes, stream)

    def status(self, stream=None) -> int:
        """Flags of the last step's device checks (0: none failed); waits for the stream."""
        return B.rkv_device_status(self.workspace, stream)

    def device_status(self, stream=None) -> int:
        """Flags of the last rkv_step_device call's device checks."""
        return B.rkv_device_status(self.dev_ws, stream)

    def __call__(self, cache: B.rkv_cache, q_window, seq_lens: np.ndarray, stream=None) -> None:
        """score, select, compact as three calls; seq_lens (int32 numpy) is updated in place."""
        self.score(cache, q_window, seq_lens, stream)
        self.select(seq_lens, stream)
        self.compact(cache, seq_lens, stream)

    def device(self, cache: B.rkv_cache, q_window, d_seq_lens, stream=None) -> None:
        """The step through rkv_step_device: lengths in the device int32 tensor
        d_seq_lens (updated there), self.max_len as the launch bound, freed-block
        counts in the device tensor self.d_free_counts.  Capturable in a graph."""
        import torch
        if getattr(self, "dev_ws", None) is None:
            self.dev_ws_bytes = max(256, B.rkv_step_device_workspace_size(
                self.cfg, self.num_seqs, self.max_len))
            self.dev_ws = torch.empty(self.dev_ws_bytes, dtype=torch.uint8,
                                      device=self.scores.device)
            self.d_free_counts = torch.zeros(max(1, self.num_seqs), dtype=torch.int32,
                                             device=self.scores.device)
        B.rkv_step_device(self.cfg, cache, q_window, self.num_seqs, d_seq_lens, self.max_len,
                          self.scores, self.max_len, self.keep, self.free_blocks,
                          self.free_capacity, self.d_free_counts, self.dev_ws,
                          self.dev_ws_bytes, stream)

    def fused(self, cache: B.rkv_cache, q_window, seq_lens: np.ndarray, stream=None) -> None:
        """The same step through the single rkv_step call."""
        B.rkv_step(self.cfg, cache, q_window, self.num_seqs, seq_lens, self.scores, self.max_len,
                   self.keep, self.free_blocks, self.free_capacity, self.free_counts,
                   self.workspace, self.ws_bytes, stream)
