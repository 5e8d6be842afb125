"""Pins of the fp64 oracle's recurrences against things other than itself.

* brute force: the whole trajectory as a product of augmented Kronecker-form
  linear maps (a different formulation from the oracle's per-step code);
* exact rational arithmetic on dyadic (float32) inputs with the published
  Gated DeltaNet closed form S_t = a S (I - b k k^T) + b v k^T;
* closed-form special cases (alpha = 1 running sum, alpha = 0, beta = 0 pure
  decay, beta = 1 with a unit key writing the slot exactly).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ReplayOracle, widen, mamba2_step, gdn_step
from synth import get_workload, initial_state, stack_decode_inputs


def _tiny(kind, **kw):
    base = dict(batch=1, n_heads=2, n_qk_heads=1 if kind == "gdn" else 2, dv=2, dk=3,
                in_dtype="fp32", L=64, t_max=1, capacity=64, decode_steps=12,
                verify_steps=0, read_copy="none")
    base.update(kw)
    return get_workload("m2_tiny").replace(name="pin", kind=kind, **base)


def _run_oracle(wl, steps):
    seqs = [0]
    S0 = initial_state(wl, seqs)
    inp = stack_decode_inputs(wl, range(steps), seqs, workers=1)
    orc = ReplayOracle(wl, seqs, S0)
    ys = []
    for t in range(steps):
        ys.append(orc.decode({k: (None if v is None else v[t]) for k, v in inp.items()})[0])
    return S0[0].astype(np.float64), inp, np.array(ys), orc


def _w(a, wl):
    return widen(a, wl.in_dtype)


def _kron_map(kind, alpha, beta, v, k):
    """Augmented map on [vec_rowmajor(S); 1] for one head and one record."""
    P, N = len(v), len(k)
    if kind == "mamba2":
        lin = alpha * np.eye(P * N)
        off = np.outer(v, k).reshape(-1)
    else:
        M = alpha * (np.eye(N) - beta * np.outer(k, k))        # S <- S M + b v k^T
        lin = np.kron(np.eye(P), M.T)
        off = (beta * np.outer(v, k)).reshape(-1)
    A = np.zeros((P * N + 1, P * N + 1))
    A[:-1, :-1] = lin
    A[:-1, -1] = off
    A[-1, -1] = 1.0
    return A


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_kronecker_unrolling(kind):
    wl = _tiny(kind)
    steps = 12
    S0, inp, ys, orc = _run_oracle(wl, steps)
    H, G = wl.n_heads, wl.n_qk_heads
    for h in range(H):
        g = h // (H // G)
        Mtot = np.eye(wl.dv * wl.dk + 1)
        for t in range(steps):
            a = _w(inp["alpha"][t, 0, h], wl)
            b = _w(inp["beta"][t, 0, h], wl) if kind == "gdn" else 0.0
            v = _w(inp["v"][t, 0, h], wl)
            k = _w(inp["k"][t, 0, g], wl)
            q = _w(inp["q"][t, 0, g], wl)
            Mtot = _kron_map(kind, a, b, v, k) @ Mtot
            St = (Mtot @ np.append(S0[h].reshape(-1), 1.0))[:-1].reshape(wl.dv, wl.dk)
            np.testing.assert_allclose(ys[t, h], St @ q, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(orc.S[0, h], St, rtol=1e-12, atol=1e-13)


def _frac(x):
    return Fraction(float(x))


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_exact_rationals(kind):
    """fp64 oracle within 1e-13 of the exact trajectory (inputs are dyadic)."""
    wl = _tiny(kind, n_heads=1, n_qk_heads=1, dv=2, dk=4, decode_steps=20)
    steps = 20
    S0, inp, ys, orc = _run_oracle(wl, steps)
    P, N = wl.dv, wl.dk
    S = [[_frac(S0[0][p, n]) for n in range(N)] for p in range(P)]
    for t in range(steps):
        a = _frac(_w(inp["alpha"][t, 0, 0], wl))
        b = _frac(_w(inp["beta"][t, 0, 0], wl)) if kind == "gdn" else None
        v = [_frac(x) for x in _w(inp["v"][t, 0, 0], wl)]
        k = [_frac(x) for x in _w(inp["k"][t, 0, 0], wl)]
        q = [_frac(x) for x in _w(inp["q"][t, 0, 0], wl)]
        if kind == "mamba2":
            S = [[a * S[p][n] + v[p] * k[n] for n in range(N)] for p in range(P)]
        else:
            # S (I - b k k^T) = S - b (S k) k^T
            Sk = [sum(S[p][m] * k[m] for m in range(N)) for p in range(P)]
            S = [[a * (S[p][n] - b * Sk[p] * k[n]) + b * v[p] * k[n] for n in range(N)]
                 for p in range(P)]
        y = [sum(S[p][n] * q[n] for n in range(N)) for p in range(P)]
        ref = np.array([float(x) for x in y])
        scale = max(np.max(np.abs(ref)), 1e-300)
        assert np.max(np.abs(ys[t, 0] - ref)) / scale < 1e-13
    Sref = np.array([[float(x) for x in row] for row in S])
    assert np.max(np.abs(orc.S[0, 0] - Sref)) / np.max(np.abs(Sref)) < 1e-13


def _rand_head(rng, P, N):
    return rng.standard_normal((P, N))


def test_mamba2_alpha_one_is_running_sum():
    rng = np.random.default_rng(1)
    H, P, N, T = 3, 4, 5, 10
    S0 = rng.standard_normal((H, P, N))
    v = rng.standard_normal((T, H, P)); k = rng.standard_normal((T, H, N)); q = rng.standard_normal((T, H, N))
    cum = S0[None] + np.cumsum(v[:, :, :, None] * k[:, :, None, :], axis=0)
    S = S0.copy()
    for t in range(T):
        S, y = mamba2_step(S, np.ones(H), v[t], k[t], q[t])
        ref = np.einsum("hpn,hn->hp", cum[t], q[t])
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_mamba2_alpha_zero_forgets():
    rng = np.random.default_rng(2)
    H, P, N = 2, 3, 4
    S = rng.standard_normal((H, P, N))
    v = rng.standard_normal((H, P)); k = rng.standard_normal((H, N)); q = rng.standard_normal((H, N))
    _, y = mamba2_step(S, np.zeros(H), v, k, q)
    np.testing.assert_allclose(y, v * (k * q).sum(-1)[:, None], rtol=1e-14)


def test_gdn_beta_zero_is_pure_decay():
    rng = np.random.default_rng(3)
    H, P, N = 2, 3, 4
    S0 = rng.standard_normal((H, P, N))
    S = S0.copy()
    G = np.ones(H)
    for t in range(6):
        a = rng.uniform(0.5, 1.0, H)
        G = G * a
        q = rng.standard_normal((H, N))
        S, o = gdn_step(S, a, np.zeros(H), rng.standard_normal((H, P)), rng.standard_normal((H, N)), q)
        np.testing.assert_allclose(o, G[:, None] * np.einsum("hpn,hn->hp", S0, q), rtol=1e-13)


def test_gdn_beta_one_unit_key_writes_slot():
    """With b = 1 and |k| = 1 the delta rule stores v under key k: S_t k = v, and q = k reads v."""
    rng = np.random.default_rng(4)
    H, P, N = 2, 3, 4
    S = rng.standard_normal((H, P, N))
    for t in range(5):
        k = np.zeros((H, N)); k[:, t % N] = 1.0                # exactly unit keys
        v = rng.standard_normal((H, P))
        S, o = gdn_step(S, rng.uniform(0.3, 1.0, H), np.ones(H), v, k, k.copy())
        np.testing.assert_allclose(np.einsum("hpn,hn->hp", S, k), v, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(o, v, rtol=1e-14, atol=1e-14)
    k = np.array([[0.6, 0.8, 0.0, 0.0]] * H)                   # unit norm, not a basis vector
    v = rng.standard_normal((H, P))
    S, o = gdn_step(S, np.full(H, 0.75), np.ones(H), v, k, k.copy())
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-13)


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x3E20], np.uint16)
    ref = np.array([1.0, -1.0, 2.0 ** -133, 3.3895313892515355e38, 0.15625])
    np.testing.assert_array_equal(widen(bits, "bf16"), ref)
