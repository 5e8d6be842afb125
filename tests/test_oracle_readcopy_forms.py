"""The oracle's read-copy rule against the window-unrolled replay forms (CPU).

Page 1, section on what got faster (low-precision paragraph), and page 4 "What
shipped" (quantisation paragraph): a low-precision copy of the checkpoint serves
the reads while the full-precision checkpoint drives the recurrence.  Page 4
"What shipped" (unrolling paragraph): a non-flush output is the decayed
checkpoint applied to the query plus a sum over the buffered records.

Together these fix every non-flush read-copy output: it is the replay form of
the window evaluated on the dequantised copy of the last folded checkpoint.
The oracle computes it differently, as a stepwise chain restarted from the
dequantised copy at every fold; these tests hold the two to 1e-12 (normwise)
for fp8 and MXFP4 copies, with the Mamba-2 replay formula and, for Gated
DeltaNet and KDA, the query-transform sweep.  Flush-step outputs must equal
the full-precision recurrence.  The quantisers themselves are pinned in
tests/test_oracle_quant.py.
"""
import numpy as np
import pytest

from oracle import ReplayOracle, read_copy_dequant, replay_forms as rf, widen
from synth import accept_counts, decode_inputs, draft_inputs, get_workload, initial_state


def _wl(kind, fmt, dtype):
    base = {"mamba2": "m2_readcopy_b256", "gdn": "gdn_b256", "kda": "kda_b256"}[kind]
    shape = {"mamba2": dict(n_heads=3, n_qk_heads=3), "gdn": dict(n_heads=4, n_qk_heads=2),
             "kda": dict(n_heads=2, n_qk_heads=2)}[kind]
    return get_workload(base).replace(name="rcf", batch=2, dv=12, dk=64, in_dtype=dtype, L=5, t_max=1,
                                      capacity=5, read_copy=fmt, **shape)


def _rel(x, ref):
    return np.max(np.abs(x - ref), axis=-1) / np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)


def _window_output(kind, S_read, recs, q):
    """Replay form for one value head over the window records (oldest first)."""
    if kind == "mamba2":
        return rf.m2_replay_output(S_read, recs, q)
    if kind == "gdn":
        return rf.query_transform_output(S_read, recs, q, "gdn")
    return rf.kda_query_transform_output(S_read, recs, q)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_read_copy_outputs_equal_replay_of_dequantised_checkpoint(kind, fmt, dtype):
    wl = _wl(kind, fmt, dtype)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    exact = ReplayOracle(wl.replace(read_copy="none"), seqs, S0)
    grp = wl.n_heads // wl.n_qk_heads
    # the copy the outputs read: quantised from the float32 checkpoint at init and at each fold
    S_read = read_copy_dequant(fmt, S0)
    window = [[] for _ in seqs]
    checked = 0
    for t in range(13):
        inp = decode_inputs(wl, t, seqs)
        y = orc.decode(inp)
        y_full = exact.decode(inp)
        flush = (t + 1) % wl.L == 0
        for i in range(wl.batch):
            rec = {f: (None if inp[f] is None else widen(inp[f][i], wl.in_dtype))
                   for f in ("alpha", "beta", "v", "k", "q")}
            window[i].append(rec)
            if flush:
                assert np.max(_rel(y[i], y_full[i])) == 0.0, f"flush step {t} must read the fp32 state"
                continue
            for h in range(wl.n_heads):
                g = h // grp
                recs = [dict(alpha=r["alpha"][h], beta=None if r["beta"] is None else r["beta"][h],
                             v=r["v"][h], k=r["k"][g]) for r in window[i]]
                want = _window_output(kind, S_read[i, h], recs, rec["q"][g])
                err = _rel(y[i, h], want)
                assert err < 1e-12, f"step {t} seq {i} head {h}: {err:.3g}"
                checked += 1
        if flush:
            S_read = read_copy_dequant(fmt, exact.S.astype(np.float32))
            window = [[] for _ in seqs]
        assert np.max(_rel(orc.y_exact, y_full)) == 0.0
    assert checked == 11 * wl.batch * wl.n_heads        # 13 steps, folds at steps 4 and 9


def test_read_copy_outputs_differ_from_the_fp32_outputs():
    """The rule is not vacuous: a non-flush read-copy output is not the fp32 output."""
    wl = _wl("mamba2", "mxfp4", "fp32")
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    inp = decode_inputs(wl, 0, seqs)
    y = orc.decode(inp)
    assert np.min(_rel(y, orc.y_exact)) > 1e-4


def _recs_of(inp, i, dtype, t=None):
    return {f: (None if inp[f] is None else widen(inp[f][i] if t is None else inp[f][i, t], dtype))
            for f in ("alpha", "beta", "v", "k", "q")}


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("kind", ["mamba2", "gdn", "kda"])
def test_read_copy_window_holds_committed_drafts(kind, fmt):
    """Accepted drafts join the window like decode records: after verify / commit rounds
    with a per-sequence accepted prefix, every non-flush decode output is the replay form
    over all records committed since the last fold (drafts and decode records, oldest
    first) on the dequantised copy of the checkpoint."""
    wl = _wl(kind, fmt, "bf16").replace(L=8, capacity=10, t_max=3)
    seqs = list(range(wl.batch))
    S0 = initial_state(wl, seqs)
    orc = ReplayOracle(wl, seqs, S0)
    grp = wl.n_heads // wl.n_qk_heads
    S_read = [read_copy_dequant(fmt, S0[i]) for i in seqs]
    window = [[] for _ in seqs]
    for r in range(2):                      # two rounds: up to 6 drafts, at most 7 records
        d = draft_inputs(wl, r, seqs, 3)
        orc.verify(d, 3)
        acc = accept_counts(wl, r, 3)[: wl.batch]
        acc[0] = 3                           # sequence 0 takes every draft
        orc.commit(acc, 3)
        for i in seqs:
            window[i] += [_recs_of(d, i, wl.in_dtype, t)
                          for t in range(int(acc[i]))]
    assert not orc.err and len(window[0]) == 6
    checked = 0
    for t in range(10):
        h_before = orc.h().copy()
        inp = decode_inputs(wl, t, seqs)
        y = orc.decode(inp)
        for i in seqs:
            rec = _recs_of(inp, i, wl.in_dtype)
            window[i].append(rec)
            if h_before[i] + 1 >= wl.L:        # fold step: a new copy of the new checkpoint
                S_read[i] = read_copy_dequant(fmt, orc.S_ckpt[i].astype(np.float32))
                window[i] = []
                continue
            for h in range(wl.n_heads):
                g = h // grp
                recs = [dict(alpha=x["alpha"][h], beta=None if x["beta"] is None else x["beta"][h],
                             v=x["v"][h], k=x["k"][g]) for x in window[i]]
                want = _window_output(kind, S_read[i][h], recs, rec["q"][g])
                err = _rel(y[i, h], want)
                assert err < 1e-12, f"step {t} seq {i} head {h}: {err:.3g}"
                checked += 1
    assert checked > 0 and not orc.err
