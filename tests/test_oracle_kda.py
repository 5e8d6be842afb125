"""Pins of the oracle's KDA recurrence (per-key-channel gated delta rule).

The pages name Kimi Delta Attention as an SSM layer and say the replay reframing
carries over to its delta-rule update (page 4, "Why it matters") but give no
formula; the oracle follows KDA's publication (Kimi Linear):
S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t.
These tests pin the oracle's code against that formula through other routes:

* brute force: the trajectory as a product of augmented Kronecker-form maps;
* exact rational arithmetic on the dyadic (float32) inputs;
* special cases: a gate constant over channels is the Gated DeltaNet step;
  b = 0 is a pure per-channel decay S_0 Diag(prod a); b = 1 with a unit key
  stores v under that key exactly;
* the window forms: the query-transform output equals the stepwise recurrence;
* rollback: verify(T) + commit(a) equals decoding only the accepted records.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ReplayOracle, widen, kda_step, gdn_step, replay_forms as rf
from synth import (get_workload, initial_state, stack_decode_inputs, stack_draft_inputs,
                   accept_counts)


def _tiny(**kw):
    base = dict(batch=1, n_heads=2, n_qk_heads=1, dv=2, dk=3, in_dtype="fp32", L=64, t_max=1,
                capacity=64, decode_steps=12, verify_steps=0, read_copy="none")
    base.update(kw)
    return get_workload("kda_b256").replace(name="pin", **base)


def _run(wl, steps):
    seqs = [0]
    S0 = initial_state(wl, seqs)
    inp = stack_decode_inputs(wl, range(steps), seqs, workers=1)
    orc = ReplayOracle(wl, seqs, S0)
    ys = [orc.decode({k: (None if v is None else v[t]) for k, v in inp.items()})[0] for t in range(steps)]
    return S0[0].astype(np.float64), inp, np.array(ys), orc


def test_inputs_have_channel_gates():
    wl = _tiny(dk=8)
    inp = stack_decode_inputs(wl, range(3), [0], workers=1)
    a = widen(inp["alpha"], "fp32")
    assert a.shape == (3, 1, wl.n_heads, wl.dk)
    assert np.all((a > np.exp(-0.5) - 1e-6) & (a <= 1.0))
    assert len(np.unique(a[0, 0, 0])) > 1            # gates differ across channels


def test_kronecker_unrolling():
    wl = _tiny()
    steps = 12
    S0, inp, ys, orc = _run(wl, steps)
    H, G, P, N = wl.n_heads, wl.n_qk_heads, wl.dv, wl.dk
    for h in range(H):
        g = h // (H // G)
        Mtot = np.eye(P * N + 1)
        for t in range(steps):
            a = widen(inp["alpha"][t, 0, h], "fp32")
            b = widen(inp["beta"][t, 0, h], "fp32")
            v = widen(inp["v"][t, 0, h], "fp32")
            k = widen(inp["k"][t, 0, g], "fp32")
            q = widen(inp["q"][t, 0, g], "fp32")
            M = np.diag(a) @ (np.eye(N) - b * np.outer(k, k))      # S <- S M + b v k^T
            A = np.eye(P * N + 1)
            A[:-1, :-1] = np.kron(np.eye(P), M.T)
            A[:-1, -1] = (b * np.outer(v, k)).reshape(-1)
            Mtot = A @ Mtot
            St = (Mtot @ np.append(S0[h].reshape(-1), 1.0))[:-1].reshape(P, N)
            np.testing.assert_allclose(ys[t, h], St @ q, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(orc.S[0, h], St, rtol=1e-12, atol=1e-13)


def test_exact_rationals():
    wl = _tiny(n_heads=1, n_qk_heads=1, dv=2, dk=4, decode_steps=20)
    steps = 20
    S0, inp, ys, orc = _run(wl, steps)
    P, N = wl.dv, wl.dk
    F = lambda x: Fraction(float(x))
    S = [[F(S0[0][p, n]) for n in range(N)] for p in range(P)]
    for t in range(steps):
        a = [F(x) for x in widen(inp["alpha"][t, 0, 0], "fp32")]
        b = F(widen(inp["beta"][t, 0, 0], "fp32"))
        v = [F(x) for x in widen(inp["v"][t, 0, 0], "fp32")]
        k = [F(x) for x in widen(inp["k"][t, 0, 0], "fp32")]
        q = [F(x) for x in widen(inp["q"][t, 0, 0], "fp32")]
        # S Diag(a) (I - b k k^T) + b v k^T, expanded entry by entry
        Sd = [[S[p][n] * a[n] for n in range(N)] for p in range(P)]
        Sk = [sum(Sd[p][m] * k[m] for m in range(N)) for p in range(P)]
        S = [[Sd[p][n] - b * Sk[p] * k[n] + b * v[p] * k[n] for n in range(N)] for p in range(P)]
        ref = np.array([float(sum(S[p][n] * q[n] for n in range(N))) for p in range(P)])
        assert np.max(np.abs(ys[t, 0] - ref)) / max(np.max(np.abs(ref)), 1e-300) < 1e-13
    Sref = np.array([[float(x) for x in row] for row in S])
    assert np.max(np.abs(orc.S[0, 0] - Sref)) / np.max(np.abs(Sref)) < 1e-13


def test_constant_gate_is_gated_deltanet():
    rng = np.random.default_rng(11)
    H, P, N = 3, 4, 6
    S1 = rng.standard_normal((H, P, N))
    S2 = S1.copy()
    for _ in range(8):
        a = rng.uniform(0.5, 1.0, H)
        b = rng.uniform(0, 1, H)
        v = rng.standard_normal((H, P))
        k = rng.standard_normal((H, N)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q = rng.standard_normal((H, N))
        S1, o1 = kda_step(S1, np.repeat(a[:, None], N, axis=1), b, v, k, q)
        S2, o2 = gdn_step(S2, a, b, v, k, q)
        np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-13)


def test_beta_zero_is_channel_decay():
    rng = np.random.default_rng(12)
    H, P, N = 2, 3, 5
    S0 = rng.standard_normal((H, P, N))
    S = S0.copy()
    G = np.ones((H, N))
    for _ in range(7):
        a = rng.uniform(0.3, 1.0, (H, N))
        G = G * a
        q = rng.standard_normal((H, N))
        S, o = kda_step(S, a, np.zeros(H), rng.standard_normal((H, P)), rng.standard_normal((H, N)), q)
        np.testing.assert_allclose(o, np.einsum("hpn,hn->hp", S0, G * q), rtol=1e-13)
    np.testing.assert_allclose(S, S0 * G[:, None, :], rtol=1e-13)


def test_beta_one_unit_key_writes_slot():
    rng = np.random.default_rng(13)
    H, P, N = 2, 3, 4
    S = rng.standard_normal((H, P, N))
    for t in range(5):
        k = np.zeros((H, N)); k[:, t % N] = 1.0
        v = rng.standard_normal((H, P))
        S, o = kda_step(S, rng.uniform(0.3, 1.0, (H, N)), np.ones(H), v, k, k.copy())
        np.testing.assert_allclose(np.einsum("hpn,hn->hp", S, k), v, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(o, v, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("c", [1, 2, 7, 16, 19])
def test_query_transform_equals_stepwise(c):
    rng = np.random.default_rng(200 + c)
    P, N = 6, 10
    S0 = rng.standard_normal((P, N)) * np.sqrt(0.1)
    S = S0[None].copy()
    recs = []
    for t in range(c):
        k = rng.standard_normal(N); k /= np.linalg.norm(k)
        q = rng.standard_normal(N); q /= np.linalg.norm(q)
        rec = dict(alpha=np.exp(-rng.uniform(0, 0.5, N)), beta=rng.uniform(0, 1),
                   v=rng.standard_normal(P), k=k, q=q)
        recs.append(rec)
        S, y = kda_step(S, rec["alpha"][None], np.array([rec["beta"]]), rec["v"][None], k[None], q[None])
        yq = rf.kda_query_transform_output(S0, recs, q)
        assert np.max(np.abs(yq - y[0])) / np.max(np.abs(y[0])) < 1e-12


def test_rollback_equals_never_seeing_rejected_drafts():
    wl = get_workload("kda_b256").replace(batch=3, n_heads=4, n_qk_heads=4, dv=8, dk=16)
    seqs = list(range(wl.batch))
    T = wl.t_max
    S0 = initial_state(wl, seqs)
    A = ReplayOracle(wl, seqs, S0)
    B = [ReplayOracle(wl, [i], S0[i:i + 1]) for i in seqs]
    for step in range(12):
        drafts = {k: (None if v is None else v[0])
                  for k, v in stack_draft_inputs(wl, [step], seqs, T, workers=1).items()}
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
    assert not A.err
