"""Per-step input generation in parallel over sequences (input recipe only).

A long-running run at serving batch needs one batch of inputs per step; this
splits each step's sequences over a process pool so generation keeps up, and
yields exactly the same bits as ``decode_inputs`` / ``draft_inputs``.
"""
from __future__ import annotations

from concurrent.futures import ProcessPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

from .gen import decode_inputs, draft_inputs, default_workers


def _dec(args):
    wl, step, seqs = args
    return decode_inputs(wl, step, seqs)


def _drf(args):
    wl, step, seqs, T = args
    return draft_inputs(wl, step, seqs, T)


def _cat(parts):
    out = {}
    for k in parts[0]:
        out[k] = None if parts[0][k] is None else np.concatenate([p[k] for p in parts])
    return out


class StepSource:
    """``with StepSource(wl, seqs) as src: x = src.decode(step)`` (arrays [len(seqs), ...])."""

    def __init__(self, wl, seqs: Sequence[int], workers: Optional[int] = None):
        self.wl = wl
        self.seqs = list(seqs)
        self.workers = default_workers() if workers is None else workers
        n = max(1, min(self.workers, len(self.seqs)))
        step = -(-len(self.seqs) // n)
        self.chunks: List[List[int]] = [self.seqs[i:i + step] for i in range(0, len(self.seqs), step)]
        self.pool = ProcessPoolExecutor(max_workers=n) if n > 1 else None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def close(self):
        if self.pool is not None:
            self.pool.shutdown()
            self.pool = None

    def decode(self, step: int):
        jobs = [(self.wl, step, c) for c in self.chunks]
        if self.pool is None:
            return _cat([_dec(j) for j in jobs])
        return _cat(list(self.pool.map(_dec, jobs)))

    def drafts(self, step: int, T: int):
        jobs = [(self.wl, step, c, T) for c in self.chunks]
        if self.pool is None:
            return _cat([_drf(j) for j in jobs])
        return _cat(list(self.pool.map(_drf, jobs)))
