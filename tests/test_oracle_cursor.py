"""Pins of the oracle's integer cursor policy and the rollback invariant.

Page 4 "What shipped": the window holds 16 records and is folded when full;
speculative drafts go into the buffer, acceptance moves the cursor forward, and
any record beyond the cursor is dead and will simply be written over later.
Page 1 (what got faster): rollback needs neither snapshots nor a state restore.
"""
import json
import os

import numpy as np
import pytest

from oracle import ReplayOracle
from synth import (get_workload, initial_state, stack_decode_inputs, stack_draft_inputs,
                   accept_counts)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLD, "page_facts.json")) as f:
        return json.load(f)


def _sl(d, t):
    return {k: (None if v is None else v[t]) for k, v in d.items()}


def test_tiny_workload_flushes_four_times():
    wl = get_workload("m2_tiny")
    facts = _facts()
    assert wl.L == facts["window_L"]
    orc = ReplayOracle(wl, range(wl.batch), track_state=False)
    inp = stack_decode_inputs(wl, range(wl.decode_steps), range(wl.batch), workers=1)
    flush_steps = []
    for t in range(wl.decode_steps):
        before = orc.n_ckpt.copy()
        orc.decode(_sl(inp, t))
        assert np.all(orc.n_committed == t + 1)
        assert np.all(orc.n_ckpt == 16 * ((t + 1) // 16))
        if np.any(orc.n_ckpt != before):
            flush_steps.append(t + 1)
    assert flush_steps == [16, 32, 48, 64]


def test_state_bytes_match_page():
    """One Mamba-2 layer at the serving shape holds 4 MiB of fp32 state per sequence."""
    wl = get_workload("m2_decode_b256")
    assert wl.n_heads * wl.dv * wl.dk * 4 == _facts()["state_bytes_per_sequence_layer_fp32"]


def test_l1_every_step_flushes_and_checkpoint_is_state():
    wl = get_workload("m2_tiny").replace(L=1, capacity=1)
    seqs = [0, 1]
    orc = ReplayOracle(wl, seqs, initial_state(wl, seqs))
    inp = stack_decode_inputs(wl, range(5), seqs, workers=1)
    for t in range(5):
        orc.decode(_sl(inp, t))
        assert np.all(orc.n_ckpt == orc.n_committed)
        np.testing.assert_array_equal(orc.S_ckpt, orc.S)


@pytest.mark.parametrize("name", ["m2_verify_b512", "gdn_b256"])
def test_rollback_equals_never_seeing_rejected_drafts(name):
    """verify(T) + commit(a) leaves exactly the state, cursor and live ring of appending a records."""
    wl = get_workload(name).replace(batch=3, n_heads=4, n_qk_heads=2 if name.startswith("gdn") else 4,
                                    dv=8, dk=16)
    seqs = list(range(wl.batch))
    T = wl.t_max
    S0 = initial_state(wl, seqs)
    A = ReplayOracle(wl, seqs, S0)
    # reference: one oracle per sequence that only ever sees the accepted drafts, as decode steps
    B = [ReplayOracle(wl, [i], S0[i:i + 1]) for i in seqs]
    for step in range(12):
        drafts = _sl(stack_draft_inputs(wl, [step], seqs, T, workers=1), 0)
        acc = accept_counts(wl, step, T)[: wl.batch]
        A.verify(drafts, T)
        A.commit(acc, T)
        A.flush(wl.L)
        for i in seqs:
            for t in range(int(acc[i])):
                B[i].decode({k: (None if v is None else v[i:i + 1, t]) for k, v in drafts.items()})
            B[i].flush(wl.L)
            assert A.n_committed[i] == B[i].n_committed[0]
            np.testing.assert_array_equal(A.S[i], B[i].S[0])
            # A folds after commit, B when the window fills: compare the newest records live in both
            la, lb = A.live_slots(i), B[i].live_slots(0)
            n = min(len(la), len(lb))
            for f in ("alpha", "v", "k", "q"):
                for sa, sb in zip(la[len(la) - n:], lb[len(lb) - n:]):
                    np.testing.assert_array_equal(A.ring[f][i, sa], B[i].ring[f][0, sb])
    assert not A.err and not any(b.err for b in B)


def test_verify_overflow_sets_error_and_leaves_sequence():
    wl = get_workload("m2_verify_b512").replace(batch=2, n_heads=2, n_qk_heads=2, dv=4, dk=8)
    seqs = [0, 1]
    orc = ReplayOracle(wl, seqs, initial_state(wl, seqs))
    T = wl.t_max
    # commit without flushing until h + T > C for sequence 0
    for step in range(4):
        d = _sl(stack_draft_inputs(wl, [step], seqs, T, workers=1), 0)
        orc.verify(d, T)
        orc.commit(np.array([T, 0], np.int32), T)
    assert orc.h()[0] == 16 and not orc.err
    S_before = orc.S.copy()
    d = _sl(stack_draft_inputs(wl, [9], seqs, T, workers=1), 0)
    O = orc.verify(d, T)
    assert orc.err
    assert np.all(np.isnan(O[0])) and np.all(np.isfinite(O[1]))
    orc.commit(np.array([T, 1], np.int32), T)
    np.testing.assert_array_equal(orc.S[0], S_before[0])
    assert orc.n_committed[0] == 16 and orc.n_committed[1] == 1


def test_commit_out_of_range_sets_error():
    wl = get_workload("m2_verify_b512").replace(batch=2, n_heads=2, n_qk_heads=2, dv=4, dk=8)
    seqs = [0, 1]
    orc = ReplayOracle(wl, seqs, initial_state(wl, seqs))
    d = _sl(stack_draft_inputs(wl, [0], seqs, 4, workers=1), 0)
    orc.verify(d, 2)
    orc.commit(np.array([3, 2], np.int32), 2)
    assert orc.err
    assert list(orc.n_committed) == [0, 2]


def test_read_copy_never_feeds_recurrence():
    """The fp32 state trajectory is identical with and without a read copy."""
    base = get_workload("m2_tiny").replace(decode_steps=40)
    seqs = [0, 1]
    S0 = initial_state(base, seqs)
    inp = stack_decode_inputs(base, range(40), seqs, workers=1)
    plain = ReplayOracle(base, seqs, S0)
    fp8 = ReplayOracle(base.replace(read_copy="fp8"), seqs, S0)
    mx = ReplayOracle(base.replace(read_copy="mxfp4"), seqs, S0)
    for t in range(40):
        y0 = plain.decode(_sl(inp, t))
        y1 = fp8.decode(_sl(inp, t))
        y2 = mx.decode(_sl(inp, t))
        np.testing.assert_array_equal(plain.S, fp8.S)
        np.testing.assert_array_equal(plain.S, mx.S)
        if (t + 1) % 16 == 0:                       # flush steps read the fp32 state
            np.testing.assert_array_equal(y0, y1)
        else:
            assert np.max(np.abs(y1 - y0)) > 0
            rel = np.max(np.abs(y1 - y0)) / np.max(np.abs(y0))
            assert rel < 5e-2
            rel2 = np.max(np.abs(y2 - y0)) / np.max(np.abs(y0))
            assert rel2 < 0.25
