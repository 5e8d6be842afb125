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
from synth import decode_inputs, get_workload, initial_state


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
