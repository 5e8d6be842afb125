"""Seeded input generator (input recipe only; no ReplaySSM arithmetic).

Every random stream is a numpy ``PCG64`` seeded by ``SeedSequence([seed, tag,
step, b])``, so any step or any subset of sequences regenerates the same bits
on its own.  Values are drawn in float64, rounded to float32 (round to nearest
even) and, for bf16 workloads, rounded again to bfloat16 (round to nearest
even on the float32 bits).  bf16 arrays are returned as their raw uint16 bits:
the stored bits *are* the input, consumed by both the oracle and the GPU path.

Distributions (per the workload descriptions):
* Mamba-2: A ~ U(-4, -1) once per head; per (sequence, step, head)
  dt ~ N(0, 1) and alpha = exp(-softplus(dt) * exp(A)); v ~ N(0, 1);
  k, q ~ N(0, 1/N) (the second parameter is the variance).
* Gated DeltaNet: alpha = exp(-U(0, 0.5)); beta ~ U(0, 1); v ~ N(0, 1);
  k, q ~ N(0, 1) then scaled to unit L2 norm (in float64, before the cast).
* KDA: as Gated DeltaNet, with alpha = exp(-U(0, 0.5)) drawn per (head, key
  channel) instead of per head.
* Initial state S0 ~ N(0, 0.1) (variance) in float32, or zero.
* Accepted draft count per (sequence, verify step) ~ U{0, ..., T}.
* Special records (``special_decode_inputs`` / ``special_draft_inputs``): the records
  above with exact special values mixed in by head and record index r: alpha 0 or 1
  (KDA: all channels 0, all 1, or alternating 0/1), beta 0 or 1, a unit basis vector as
  the key, one fixed key repeated in every record of a (sequence, key head), and q equal
  to k.
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

from .workloads import Workload

# stream tags
_TAG_HEAD = 0xA0
_TAG_S0 = 0x50
_TAG_DECODE = 0x01
_TAG_DRAFT = 0x02
_TAG_ACCEPT = 0x03
_TAG_TREE = 0x04
_TAG_SPECIAL = 0x05
_TAG_SPECIAL_KEY = 0x06


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _cast(x64: np.ndarray, in_dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if in_dtype == "fp32":
        return x32
    if in_dtype == "bf16":
        return bf16_bits_from_f32(x32)
    raise ValueError(in_dtype)


def head_params(wl: Workload) -> Dict[str, np.ndarray]:
    """Per-head constants fixed across batch and steps (Mamba-2: A ~ U(-4,-1))."""
    if wl.kind == "mamba2":
        return {"A": _rng(wl.seed, _TAG_HEAD).uniform(-4.0, -1.0, size=wl.n_heads)}
    return {}


def initial_state(wl: Workload, seqs: Sequence[int]) -> np.ndarray:
    """float32 [len(seqs), H, P, N] initial state."""
    out = np.zeros((len(seqs), wl.n_heads, wl.dv, wl.dk), np.float32)
    if wl.s0 == "zero":
        return out
    std = np.sqrt(0.1)
    for i, b in enumerate(seqs):
        out[i] = (_rng(wl.seed, _TAG_S0, b).standard_normal(
            (wl.n_heads, wl.dv, wl.dk)) * std).astype(np.float32)
    return out


def _record(wl: Workload, g: np.random.Generator, hp: Dict[str, np.ndarray]):
    """One input record for all heads of one sequence, in float64."""
    H, G, P, N = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    if wl.kind == "mamba2":
        dt = g.standard_normal(H)
        softplus = np.logaddexp(0.0, dt)
        alpha = np.exp(-softplus * np.exp(hp["A"]))
        beta = None
        v = g.standard_normal((H, P))
        k = g.standard_normal((G, N)) / np.sqrt(N)
        q = g.standard_normal((G, N)) / np.sqrt(N)
    elif wl.kind in ("gdn", "kda"):
        alpha = np.exp(-g.uniform(0.0, 0.5, size=H if wl.kind == "gdn" else (H, N)))
        beta = g.uniform(0.0, 1.0, size=H)
        v = g.standard_normal((H, P))
        k = g.standard_normal((G, N))
        q = g.standard_normal((G, N))
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    else:
        raise ValueError(wl.kind)
    return alpha, beta, v, k, q


def _fixed_key(wl: Workload, b: int, g: int) -> np.ndarray:
    """A key that repeats in every special record of (sequence b, key head g)."""
    k = _rng(wl.seed, _TAG_SPECIAL_KEY, b, g).standard_normal(wl.dk)
    return k / (np.sqrt(wl.dk) if wl.kind == "mamba2" else np.linalg.norm(k))


def _special_record(wl: Workload, g: np.random.Generator, hp, b: int, r: int):
    """Record r of sequence b with special values mixed in (float64, before the cast)."""
    alpha, beta, v, k, q = _record(wl, g, hp)
    H, G, N = wl.n_heads, wl.n_qk_heads, wl.dk
    for h in range(H):
        m = (h + r) % 4
        if wl.kind == "kda":
            if m == 0:
                alpha[h] = 0.0
            elif m == 1:
                alpha[h] = 1.0
            elif m == 2:
                alpha[h] = np.arange(N) % 2
        elif m < 2:
            alpha[h] = float(m)
        if beta is not None and (h + 2 * r) % 3 < 2:
            beta[h] = float((h + 2 * r) % 3)
    for gg in range(G):
        m = (gg + r) % 3
        if m == 0:
            k[gg] = 0.0
            k[gg, (r + gg) % N] = 1.0
        elif m == 1:
            k[gg] = _fixed_key(wl, b, gg)
        if (gg + r) % 2 == 0:
            q[gg] = k[gg]
    return alpha, beta, v, k, q


def special_decode_inputs(wl: Workload, step: int, seqs: Sequence[int]):
    """Decode inputs of one step with special values mixed in (record index r = step)."""
    hp = head_params(wl)
    out = _empty(wl, (len(seqs),))
    for i, b in enumerate(seqs):
        a, be, v, k, q = _special_record(wl, _rng(wl.seed, _TAG_SPECIAL, step, b), hp, b, step)
        _put(out, (i,), wl, a, be, v, k, q)
    return out


def special_draft_inputs(wl: Workload, step: int, seqs: Sequence[int], T: int):
    """T draft records of one verify step with special values (record index r = step * T + tau)."""
    hp = head_params(wl)
    out = _empty(wl, (len(seqs), T))
    for i, b in enumerate(seqs):
        g = _rng(wl.seed, _TAG_SPECIAL, 1 << 20, step, b)
        for t in range(T):
            a, be, v, k, q = _special_record(wl, g, hp, b, step * T + t)
            _put(out, (i, t), wl, a, be, v, k, q)
    return out


def _put(out, idx, wl, a, be, v, k, q):
    out["alpha"][idx] = _cast(a, wl.in_dtype)
    if be is not None:
        out["beta"][idx] = _cast(be, wl.in_dtype)
    out["v"][idx] = _cast(v, wl.in_dtype)
    out["k"][idx] = _cast(k, wl.in_dtype)
    out["q"][idx] = _cast(q, wl.in_dtype)


def _empty(wl: Workload, lead: tuple) -> Dict[str, Optional[np.ndarray]]:
    dt = np.float32 if wl.in_dtype == "fp32" else np.uint16
    H, G, P, N = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    return {
        "alpha": np.zeros(lead + ((H, N) if wl.kind == "kda" else (H,)), dt),
        "beta": np.zeros(lead + (H,), dt) if wl.kind in ("gdn", "kda") else None,
        "v": np.zeros(lead + (H, P), dt),
        "k": np.zeros(lead + (G, N), dt),
        "q": np.zeros(lead + (G, N), dt),
    }


def decode_inputs(wl: Workload, step: int, seqs: Sequence[int]):
    """Inputs of one decode step for sequences ``seqs`` (leading dim = len(seqs))."""
    hp = head_params(wl)
    out = _empty(wl, (len(seqs),))
    for i, b in enumerate(seqs):
        a, be, v, k, q = _record(wl, _rng(wl.seed, _TAG_DECODE, step, b), hp)
        out["alpha"][i] = _cast(a, wl.in_dtype)
        if be is not None:
            out["beta"][i] = _cast(be, wl.in_dtype)
        out["v"][i] = _cast(v, wl.in_dtype)
        out["k"][i] = _cast(k, wl.in_dtype)
        out["q"][i] = _cast(q, wl.in_dtype)
    return out


def draft_inputs(wl: Workload, step: int, seqs: Sequence[int], T: int):
    """T draft records of one verify step: arrays [len(seqs), T, ...]."""
    hp = head_params(wl)
    out = _empty(wl, (len(seqs), T))
    for i, b in enumerate(seqs):
        g = _rng(wl.seed, _TAG_DRAFT, step, b)
        for t in range(T):
            a, be, v, k, q = _record(wl, g, hp)
            out["alpha"][i, t] = _cast(a, wl.in_dtype)
            if be is not None:
                out["beta"][i, t] = _cast(be, wl.in_dtype)
            out["v"][i, t] = _cast(v, wl.in_dtype)
            out["k"][i, t] = _cast(k, wl.in_dtype)
            out["q"][i, t] = _cast(q, wl.in_dtype)
    return out


def accept_counts(wl: Workload, step: int, T: int) -> np.ndarray:
    """Accepted prefix length per sequence, U{0..T}, int32 [batch]."""
    return _rng(wl.seed, _TAG_ACCEPT, step).integers(0, T + 1, size=wl.batch).astype(np.int32)


def draft_tree(wl: Workload, step: int, T: int):
    """A random draft tree per sequence and an accepted path in it (input recipe only).

    parent int32 [batch, T]: draft t's parent is uniform over the committed head (-1) and
    the earlier drafts 0..t-1 (a random recursive tree).  path int32 [batch, T] and
    accept int32 [batch]: a uniformly chosen draft's root-to-node path, of which a prefix
    of uniform length 0..depth is accepted (entries past the accepted prefix are -1)."""
    g = _rng(wl.seed, _TAG_TREE, step)
    parent = np.empty((wl.batch, T), np.int32)
    for t in range(T):
        parent[:, t] = g.integers(-1, t, size=wl.batch)
    node = g.integers(0, T, size=wl.batch)
    path = np.full((wl.batch, T), -1, np.int32)
    accept = np.zeros(wl.batch, np.int32)
    for b in range(wl.batch):
        chain = []
        d = int(node[b])
        while d >= 0:
            chain.append(d)
            d = int(parent[b, d])
        chain.reverse()
        a = int(g.integers(0, len(chain) + 1))
        path[b, :a] = chain[:a]
        accept[b] = a
    return parent, path, accept


def _decode_job(args):
    wl, step, seqs = args
    return decode_inputs(wl, step, seqs)


def _draft_job(args):
    wl, step, seqs, T = args
    return draft_inputs(wl, step, seqs, T)


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stack(parts: List[Dict[str, Optional[np.ndarray]]]):
    out = {}
    for key in parts[0]:
        if parts[0][key] is None:
            out[key] = None
        else:
            out[key] = np.stack([p[key] for p in parts])
    return out


def stack_decode_inputs(wl: Workload, steps: Iterable[int], seqs: Sequence[int],
                        workers: Optional[int] = None):
    """Decode inputs for several steps: arrays [n_steps, len(seqs), ...]."""
    steps = list(steps)
    workers = default_workers() if workers is None else workers
    jobs = [(wl, s, list(seqs)) for s in steps]
    if workers <= 1 or len(jobs) <= 1:
        return _stack([_decode_job(j) for j in jobs])
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return _stack(list(ex.map(_decode_job, jobs)))


def stack_draft_inputs(wl: Workload, steps: Iterable[int], seqs: Sequence[int], T: int,
                       workers: Optional[int] = None):
    """Draft inputs for several verify steps: arrays [n_steps, len(seqs), T, ...]."""
    steps = list(steps)
    workers = default_workers() if workers is None else workers
    jobs = [(wl, s, list(seqs), T) for s in steps]
    if workers <= 1 or len(jobs) <= 1:
        return _stack([_draft_job(j) for j in jobs])
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return _stack(list(ex.map(_draft_job, jobs)))
