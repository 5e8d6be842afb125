"""Oracle trajectories for the GPU parity tests, one sampled sequence per worker.

Each worker regenerates its sequence's inputs from the seed (``synth``) and runs
the fp64 oracle; nothing here reads a GPU result.
"""
from __future__ import annotations

from concurrent.futures import ProcessPoolExecutor
from typing import Dict, List, Sequence

import numpy as np

from oracle import ReplayOracle
from synth import accept_counts, decode_inputs, draft_inputs, initial_state
from synth.gen import default_workers


READ_TOL = 2e-5   # the fp32-state tolerance the GPU checkpoint is held to


def _decode_seq(args):
    wl, b, steps, keep_ckpt = args
    rt = READ_TOL if wl.read_copy != "none" else None
    orc = ReplayOracle(wl, [b], initial_state(wl, [b]), read_tol=rt)
    ys, nc, nk, ck, al = [], [], [], {}, []
    for t in range(steps):
        ys.append(orc.decode(decode_inputs(wl, t, [b]))[0])
        if rt is not None:
            al.append(orc.allowance[0].copy())
        nc.append(int(orc.n_committed[0]))
        nk.append(int(orc.n_ckpt[0]))
        if nk[-1] == nc[-1] and keep_ckpt(t):
            ck[t] = orc.S_ckpt[0].copy()
    return dict(y=np.array(ys), nc=np.array(nc), nk=np.array(nk), ckpt=ck,
                allowance=np.array(al) if al else None)


def _spec_seq(args):
    wl, b, decode_steps, verify_steps, T, keep_ckpt, keep_dec = args
    orc = ReplayOracle(wl, [b], initial_state(wl, [b]))
    yd, ckd = [], {}
    for t in range(decode_steps):
        yd.append(orc.decode(decode_inputs(wl, t, [b]))[0])
        if keep_dec(t):
            ckd[t] = orc.S_ckpt[0].copy()
    O, nc, nk, ck = [], [], [], {}
    for s in range(verify_steps):
        O.append(orc.verify(draft_inputs(wl, s, [b], T), T)[0])
        orc.commit(accept_counts(wl, s, T)[b:b + 1], T)
        orc.flush(wl.L)
        nc.append(int(orc.n_committed[0]))
        nk.append(int(orc.n_ckpt[0]))
        if keep_ckpt(s):
            ck[s] = orc.S_ckpt[0].copy()
    return dict(y=np.array(yd) if yd else None, O=np.array(O), nc=np.array(nc), nk=np.array(nk),
                ckpt=ck, ckpt_decode=ckd, err=orc.err)


class _Every:
    def __init__(self, every, last):
        self.every, self.last = every, last

    def __call__(self, t):
        return t == self.last or (self.every and t % self.every == self.every - 1)


def decode_runs(wl, seqs: Sequence[int], steps: int, ckpt_every: int = 0) -> Dict[int, dict]:
    keep = _Every(ckpt_every, steps - 1)
    jobs = [(wl, b, steps, keep) for b in seqs]
    with ProcessPoolExecutor(max_workers=max(1, min(default_workers(), len(jobs)))) as ex:
        return dict(zip(seqs, ex.map(_decode_seq, jobs)))


def spec_runs(wl, seqs: Sequence[int], decode_steps: int, verify_steps: int, T: int,
              ckpt_every: int = 0) -> Dict[int, dict]:
    """Decode then verify -> commit -> flush(L) per sequence.  Checkpoints are kept every
    ckpt_every steps of each phase (and after its last step): ``ckpt`` (verify phase) and
    ``ckpt_decode`` (decode phase)."""
    keep = _Every(ckpt_every, verify_steps - 1)
    keep_dec = _Every(ckpt_every, decode_steps - 1)
    jobs = [(wl, b, decode_steps, verify_steps, T, keep, keep_dec) for b in seqs]
    with ProcessPoolExecutor(max_workers=max(1, min(default_workers(), len(jobs)))) as ex:
        return dict(zip(seqs, ex.map(_spec_seq, jobs)))


def cursor_run(wl, steps: int, verify: bool, T: int = 1, decode_steps: int = 0) -> List[tuple]:
    """Counters of every sequence (integer policy only) after each step."""
    orc = ReplayOracle(wl, range(wl.batch), track_state=False)
    out = []
    if not verify:
        for t in range(steps):
            orc.decode({})
            out.append((orc.n_committed.copy(), orc.n_ckpt.copy()))
        return out
    for t in range(decode_steps):
        orc.decode({})
    for s in range(steps):
        orc.verify({}, T)
        orc.commit(accept_counts(wl, s, T), T)
        orc.flush(wl.L)
        out.append((orc.n_committed.copy(), orc.n_ckpt.copy()))
    return out
