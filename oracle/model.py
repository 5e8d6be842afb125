"""Checkpoint + ring + cursor model of ReplaySSM, stepwise in float64 (oracle).

TEST INFRASTRUCTURE ONLY.  Pages: page 4 "What shipped" (window of L buffered
records, flush on a full buffer, drafts added to the buffer and acceptance
recorded by moving the cursor forward, records beyond the cursor dead until
written over); page 1, section on what the method does (flush writes the state
once and empties the buffer) and section on what got faster (speculative
drafts appended to the buffer; the pointer advances by the accepted count; a
low-precision copy serves reads and never re-enters the recurrence).

The oracle keeps the *conventional* state S at the committed position (the
plain definition of what every output must equal) plus the integer cursor:

* decode: the record goes to ring slot ``n_committed % C``; S advances one
  step; ``n_committed += 1``; if ``h = n_committed - n_ckpt >= L`` the step is a
  flush step: the checkpoint becomes S and ``n_ckpt = n_committed``.  The output
  is ``S_t q_t`` (post-update state).  Reading: the flush happens on the step
  that appends the L-th record, so 64 steps with L = 16 flush exactly 4 times.
* verify(T): draft tau goes to slot ``(n_committed + tau) % C``; the counters do
  not move; output tau is the stepwise recurrence over drafts 0..tau applied to
  a temporary copy of S, which is then discarded.  Requires ``h + T <= C``.
* commit(a): ``0 <= a <= T`` and ``h + T <= C`` (the verify being committed could
  append its drafts); the first ``a`` drafts advance S stepwise;
  ``n_committed += a``.  Nothing else.
* flush(min_records): sequences with ``h >= max(min_records, 1)`` make the
  checkpoint equal S and set ``n_ckpt = n_committed``.
* read copy (decode only): at init and at every flush the float32 checkpoint
  is quantised; a second stepwise chain R restarts from the dequantised copy.
  Non-flush outputs are ``R_t q_t``; flush-step outputs come from S.  R never
  feeds S.

* verify_tree / commit_tree: the drafts form a tree (parent indices, each parent an
  earlier draft or the committed head).  Output tau follows tau's root-to-node path.
  Commit takes the accepted path (a chain from the head); its records move to the
  consecutive slots past the cursor, so the committed window stays contiguous.

A contract violation (verify with ``h + T > C``, commit with ``a`` out of range)
leaves that sequence untouched and sets the sticky error flag; its outputs are
NaN here.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .recurrence import widen, step
from .quant import read_copy_dequant, read_copy_ambiguity


class OracleError(ValueError):
    pass


_FIELDS = ("alpha", "beta", "v", "k", "q")


class ReplayOracle:
    """Oracle over the sequences ``seqs`` of workload ``wl``.

    ``S0``: float32 [len(seqs), H, P, N] or None (zeros).  With
    ``track_state=False`` only the integer cursor policy runs (cheap, for checking
    counters of a whole batch).
    """

    def __init__(self, wl, seqs: Sequence[int], S0: Optional[np.ndarray] = None,
                 track_state: bool = True, read_tol: Optional[float] = None):
        if wl.n_heads % wl.n_qk_heads:
            raise OracleError("H % G != 0")
        if wl.capacity < wl.L + wl.t_max - 1:
            raise OracleError("capacity < L + t_max - 1")
        self.wl = wl
        self.seqs = list(seqs)
        nb = len(self.seqs)
        self.n_committed = np.zeros(nb, np.int64)
        self.n_ckpt = np.zeros(nb, np.int64)
        self.err = False
        self.track_state = track_state
        self.flush_count = np.zeros(nb, np.int64)
        H, G, P, N, C = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk, wl.capacity
        dt = np.float32 if wl.in_dtype == "fp32" else np.uint16
        # ring of raw stored inputs (bit-exact copies of what was appended)
        # KDA gates are per (value head, key channel); the other kinds have one per head
        a_shape = (nb, C, H, N) if wl.kind == "kda" else (nb, C, H)
        self.ring = {
            "alpha": np.zeros(a_shape, dt),
            "beta": np.zeros((nb, C, H), dt),
            "v": np.zeros((nb, C, H, P), dt),
            "k": np.zeros((nb, C, G, N), dt),
            "q": np.zeros((nb, C, G, N), dt),
        }
        self._drafts = None
        self._drafts_T = 0
        self._tree = None
        if track_state:
            if S0 is None:
                S0 = np.zeros((nb, H, P, N), np.float32)
            if S0.dtype != np.float32 or S0.shape != (nb, H, P, N):
                raise OracleError("S0 must be float32 [nb, H, P, N]")
            self.S = S0.astype(np.float64)
            self.S_ckpt = self.S.copy()
            self.R = None
            # read-copy ambiguity (Mamba-2): A bounds |dS_read| elementwise for a checkpoint that
            # agrees with S to read_tol (normwise per tile); G is the checkpoint decay since the
            # last fold, so |dy| <= G * (A |q|) per output row.
            self.read_tol = read_tol
            self.allowance = np.zeros((nb, H, P))
            if wl.read_copy != "none":
                self.R = read_copy_dequant(wl.read_copy, S0.astype(np.float32))
                if read_tol is not None:
                    if wl.kind != "mamba2":
                        raise OracleError("read-copy ambiguity is modelled for Mamba-2 only")
                    self.Ramb = np.stack([self._ambiguity(S0[i].astype(np.float64)) for i in range(nb)])
                    self.Rgam = np.ones((nb, H))

    # -- helpers ---------------------------------------------------------------
    def h(self) -> np.ndarray:
        return self.n_committed - self.n_ckpt

    def _rec(self, inp: Dict[str, Optional[np.ndarray]], i: int, t: Optional[int] = None):
        out = {}
        for f in _FIELDS:
            a = inp.get(f)
            if a is None:
                out[f] = None
                continue
            a = a[i] if t is None else a[i, t]
            out[f] = widen(a, self.wl.in_dtype)
        return out

    def _store(self, i: int, slot: int, inp, t: Optional[int] = None):
        if not self.track_state:
            return
        for f in _FIELDS:
            a = inp.get(f)
            if a is None:
                continue
            self.ring[f][i, slot] = a[i] if t is None else a[i, t]

    def _ambiguity(self, S):
        delta = self.read_tol * np.max(np.abs(S), axis=(-2, -1), keepdims=True)
        return read_copy_ambiguity(self.wl.read_copy, S.astype(np.float32), delta)

    def _read_copy_step(self, i: int, rec):
        """Advance the read copy's chain by one committed record.  A non-flush output replays
        every record committed since the last fold on top of the copy, whether it was
        committed by a decode step or as an accepted draft."""
        if self.R is None:
            return
        self.R[i], _ = step(self.wl.kind, self.R[i], rec)
        if self.read_tol is not None:
            self.Rgam[i] = self.Rgam[i] * rec["alpha"]

    def _checkpoint(self, i: int):
        self.S_ckpt[i] = self.S[i]
        if self.R is not None:
            self.R[i] = read_copy_dequant(self.wl.read_copy, self.S[i].astype(np.float32))
            if self.read_tol is not None:
                self.Ramb[i] = self._ambiguity(self.S[i])
                self.Rgam[i] = 1.0

    # -- operations ------------------------------------------------------------
    def decode(self, inp) -> np.ndarray:
        """One decode step; ``inp`` arrays have leading dim len(seqs).  Returns y [nb,H,P].

        With a read copy, non-flush outputs come from the copy's chain; ``self.y_exact``
        then holds the outputs of the full-precision recurrence for the same step (without
        one, both are the same)."""
        wl = self.wl
        nb = len(self.seqs)
        y = np.full((nb, wl.n_heads, wl.dv), np.nan)
        self.y_exact = np.full((nb, wl.n_heads, wl.dv), np.nan)
        for i in range(nb):
            slot = int(self.n_committed[i] % wl.capacity)
            self._store(i, slot, inp)
            self.n_committed[i] += 1
            flush = self.n_committed[i] - self.n_ckpt[i] >= wl.L
            if self.track_state:
                rec = self._rec(inp, i)
                self.S[i], y_full = step(wl.kind, self.S[i], rec)
                self.y_exact[i] = y_full
                if self.R is not None and not flush:
                    self.R[i], y[i] = step(wl.kind, self.R[i], rec)
                    if self.read_tol is not None:
                        self.Rgam[i] = self.Rgam[i] * rec["alpha"]
                        qh = np.repeat(np.abs(rec["q"]), wl.group, axis=0)
                        self.allowance[i] = self.Rgam[i][:, None] * np.einsum("hpn,hn->hp", self.Ramb[i], qh)
                else:
                    y[i] = y_full
                    if self.R is not None and self.read_tol is not None:
                        self.allowance[i] = 0.0
            if flush:
                self.n_ckpt[i] = self.n_committed[i]
                self.flush_count[i] += 1
                if self.track_state:
                    self._checkpoint(i)
        return y

    def verify(self, drafts, T: int) -> np.ndarray:
        """Append T drafts past the cursor; return outputs [nb, T, H, P] (state untouched)."""
        wl = self.wl
        if not 1 <= T <= wl.t_max:
            raise OracleError("T out of range")
        nb = len(self.seqs)
        O = np.full((nb, T, wl.n_heads, wl.dv), np.nan)
        self._drafts, self._drafts_T = drafts, T
        self._draft_ok = np.ones(nb, bool)
        self._tree = None
        for i in range(nb):
            if self.n_committed[i] - self.n_ckpt[i] + T > wl.capacity:
                self.err = True
                self._draft_ok[i] = False
                continue
            for t in range(T):
                self._store(i, int((self.n_committed[i] + t) % wl.capacity), drafts, t)
            if self.track_state:
                S_tmp = self.S[i].copy()
                for t in range(T):
                    S_tmp, O[i, t] = step(wl.kind, S_tmp, self._rec(drafts, i, t))
        return O

    def commit(self, accept: np.ndarray, T: int):
        """Advance the cursor by the accepted prefix length ``accept[i]`` (0..T)."""
        wl = self.wl
        if self._drafts is None:
            raise OracleError("commit without a preceding verify")
        for i in range(len(self.seqs)):
            a = int(accept[i])
            h = self.n_committed[i] - self.n_ckpt[i]
            if a < 0 or a > T or h + T > wl.capacity or not self._draft_ok[i]:
                self.err = True
                continue
            if self.track_state:
                for t in range(a):
                    rec = self._rec(self._drafts, i, t)
                    self.S[i], _ = step(wl.kind, self.S[i], rec)
                    self._read_copy_step(i, rec)
            self.n_committed[i] += a

    # -- tree-shaped drafts -------------------------------------------------------
    @staticmethod
    def tree_paths(parent_row) -> Optional[list]:
        """Root-to-node draft lists of a draft tree given as parent indices (-1: child of the
        committed head; otherwise an earlier draft), or None if the encoding is invalid."""
        paths = []
        for t, p in enumerate(parent_row):
            p = int(p)
            if p < -1 or p >= t:
                return None
            paths.append(([] if p < 0 else list(paths[p])) + [t])
        return paths

    def verify_tree(self, drafts, T: int, parent: np.ndarray) -> np.ndarray:
        """Append T tree-shaped drafts past the cursor (draft tau at slot n_committed + tau,
        as in verify); output tau is the stepwise recurrence over the drafts on tau's
        root-to-node path, applied to a temporary copy of S.  ``parent`` int [nb, T]."""
        wl = self.wl
        if not 1 <= T <= wl.t_max:
            raise OracleError("T out of range")
        nb = len(self.seqs)
        O = np.full((nb, T, wl.n_heads, wl.dv), np.nan)
        self._drafts, self._drafts_T = drafts, T
        self._draft_ok = np.ones(nb, bool)
        self._tree = np.asarray(parent)
        for i in range(nb):
            paths = self.tree_paths(self._tree[i, :T])
            if paths is None or self.n_committed[i] - self.n_ckpt[i] + T > wl.capacity:
                self.err = True
                self._draft_ok[i] = False
                continue
            for t in range(T):
                self._store(i, int((self.n_committed[i] + t) % wl.capacity), drafts, t)
            if self.track_state:
                for t in range(T):
                    S_tmp = self.S[i].copy()
                    for d in paths[t]:
                        S_tmp, y = step(wl.kind, S_tmp, self._rec(drafts, i, d))
                    O[i, t] = y
        return O

    def commit_tree(self, path: np.ndarray, accept: np.ndarray, T: int):
        """Commit the accepted path of the last tree verify: path int [nb, T], its first
        accept[i] entries a chain from the committed head (path[0] a root draft, each next
        one a child of the previous).  The accepted drafts advance S in path order and their
        records move to the consecutive slots n_committed + 0..a-1; then n_committed += a."""
        wl = self.wl
        if self._drafts is None or getattr(self, "_tree", None) is None:
            raise OracleError("commit_tree without a preceding verify_tree")
        C = wl.capacity
        for i in range(len(self.seqs)):
            a = int(accept[i])
            h = self.n_committed[i] - self.n_ckpt[i]
            ok = 0 <= a <= T and h + T <= C and self._draft_ok[i]
            if ok:
                prev = -1
                for j in range(a):
                    d = int(path[i, j])
                    if not (0 <= d < T) or int(self._tree[i, d]) != prev:
                        ok = False
                        break
                    prev = d
            if not ok:
                self.err = True
                continue
            nc = int(self.n_committed[i])
            chosen = [int(path[i, j]) for j in range(a)]
            if self.track_state:
                recs = {f: self.ring[f][i].copy() for f in _FIELDS}
                for j, d in enumerate(chosen):
                    for f in _FIELDS:
                        self.ring[f][i, (nc + j) % C] = recs[f][(nc + d) % C]
                for d in chosen:
                    rec = self._rec(self._drafts, i, d)
                    self.S[i], _ = step(wl.kind, self.S[i], rec)
                    self._read_copy_step(i, rec)
            self.n_committed[i] += a

    def flush(self, min_records: int):
        """Fold sequences holding at least max(min_records, 1) records."""
        thr = max(int(min_records), 1)
        for i in range(len(self.seqs)):
            if self.n_committed[i] - self.n_ckpt[i] >= thr:
                self.n_ckpt[i] = self.n_committed[i]
                self.flush_count[i] += 1
                if self.track_state:
                    self._checkpoint(i)

    def live_slots(self, i: int):
        """Ring slots holding the committed records since the checkpoint, oldest first."""
        C = self.wl.capacity
        return [int((self.n_ckpt[i] + j) % C) for j in range(int(self.n_committed[i] - self.n_ckpt[i]))]
