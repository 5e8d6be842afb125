"""The window-unrolled forms equal the stepwise recurrence (oracle self-check).

Page 4 "What shipped": unrolling the recurrence over a window; output-only
replay on non-flush steps; flush folds the records into the checkpoint; verify
as O = S_ckpt Q D + V (W o K^T Q) with a small triangular solve on the delta
rule path.  Outputs equal conventional decoding up to floating-point error
(page 1, what the method does; page 4, same section).
"""
import numpy as np
import pytest

from oracle import mamba2_step, gdn_step, replay_forms as rf


def _records(kind, rng, c, P, N):
    recs = []
    for _ in range(c):
        k = rng.standard_normal(N)
        q = rng.standard_normal(N)
        if kind == "gdn":
            k /= np.linalg.norm(k)
            q /= np.linalg.norm(q)
            a = np.exp(-rng.uniform(0, 0.5))
        else:
            k /= np.sqrt(N)
            q /= np.sqrt(N)
            a = rng.uniform(0.3, 1.0)
        recs.append(dict(alpha=a, beta=rng.uniform(0, 1), v=rng.standard_normal(P), k=k, q=q))
    return recs


def _stepwise(kind, S0, recs):
    S = S0[None].copy()
    outs = []
    for r in recs:
        a = np.array([r["alpha"]])
        if kind == "mamba2":
            S, y = mamba2_step(S, a, r["v"][None], r["k"][None], r["q"][None])
        else:
            S, y = gdn_step(S, a, np.array([r["beta"]]), r["v"][None], r["k"][None], r["q"][None])
        outs.append(y[0])
    return S[0], outs


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("c", [1, 2, 7, 16, 19])
def test_replay_output_and_fold(kind, c):
    rng = np.random.default_rng(100 + c)
    P, N = 6, 10
    S0 = rng.standard_normal((P, N)) * np.sqrt(0.1)
    recs = _records(kind, rng, c, P, N)
    S_ref, outs = _stepwise(kind, S0, recs)
    for t in range(c):
        y = rf.query_transform_output(S0, recs[: t + 1], recs[t]["q"], kind)
        assert _rel(y, outs[t]) < 1e-12
        if kind == "mamba2":
            assert _rel(rf.m2_replay_output(S0, recs[: t + 1], recs[t]["q"]), outs[t]) < 1e-12
    fold = rf.m2_fold(S0, recs) if kind == "mamba2" else rf.gdn_fold(S0, recs)
    assert _rel(fold, S_ref) < 1e-12


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("h,T", [(0, 1), (0, 4), (5, 4), (15, 4), (3, 1)])
def test_chunk_verify(kind, h, T):
    rng = np.random.default_rng(7 * h + T)
    P, N = 5, 8
    S0 = rng.standard_normal((P, N))
    recs = _records(kind, rng, h + T, P, N)
    _, outs = _stepwise(kind, S0, recs)
    O = rf.chunk_verify(S0, recs[:h], recs[h:], [r["q"] for r in recs[h:]], kind)
    for tau in range(T):
        assert _rel(O[tau], outs[h + tau]) < 1e-12


def test_decay_matrix_is_causal():
    a = np.array([0.5, 0.25, 2.0])
    D = rf.decay_matrix(a)
    np.testing.assert_array_equal(D, [[1, 0.25, 0.5], [0, 1, 2.0], [0, 0, 1]])
