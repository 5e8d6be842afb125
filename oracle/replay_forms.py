"""Window-unrolled forms of the recurrences, one head at a time, float64 (oracle).

TEST INFRASTRUCTURE ONLY, and not used for parity: these are the algebraic
rewrites the pages describe, checked in ``tests/test_oracle_forms.py`` against
the stepwise recurrence (the definition).  A record is a dict with scalars
``alpha``, ``beta`` and vectors ``v`` [P], ``k`` [N]; records are oldest first.

* Page 4 "What shipped", unrolling paragraph: the state after a window equals the
  decayed checkpoint plus a decayed sum over the buffered (alpha, v, k) records.
  With G_t = prod_{i<=t} alpha_i (product over the records since the checkpoint)
  and decay(j -> t) = prod_{j<i<=t} alpha_i:
      S_t = G_t S_0 + sum_{j<=t} decay(j -> t) v_j k_j^T.
  Output-only (non-flush) replay: y_t = G_t S_0 q_t + sum_j decay(j -> t) (k_j . q_t) v_j.
* Page 4 "What shipped", verify paragraph: O = S_0 Q D + V (W o (K^T Q)), D the
  cumulative decay at each draft, W the causally masked decay matrix; on the
  delta-rule path the values become pseudo-values from a small triangular
  solve.  Reading: K, V span the buffer plus the drafts; D = diag(G at each
  draft); W[j, tau] = decay(j -> draft tau) for j <= draft tau, else 0.
* Gated DeltaNet pseudo-values (reading): with u_j = b_j (v_j - a_j S_{j-1} k_j),
  S_t = G_t S_0 + sum_j decay(j -> t) u_j k_j^T, and U solves the unit
  lower-triangular system u_j + sum_{i<j} b_j decay(i -> j)(k_i . k_j) u_i
  = b_j (v_j - G_j S_0 k_j).
* Query-transform form for one output (derived; equivalent): r <- q, acc <- 0;
  for i from the newest record down: c = k_i . r; acc += decay(i -> t) b_i c v_i;
  r <- r - b_i c k_i; then o_t = acc + G_t S_0 r.  Mamba-2 is the case without
  the r update and with b_i = 1 in acc.
* KDA (reading, derived the same way): with the per-channel gate a_i (a vector),
  S_i r = S_{i-1} Diag(a_i)(r - b_i (k_i . r) k_i) + b_i (k_i . r) v_i, so the sweep
  is c = b_i (k_i . r); acc += c v_i; r <- a_i o (r - c k_i), and o_t = acc + S_0 r.
  The decays ride on r, so no scalar G or decay(i -> t) appears.
"""
from __future__ import annotations

from typing import List

import numpy as np


def _alphas(recs) -> np.ndarray:
    return np.array([r["alpha"] for r in recs], np.float64)


def decay_matrix(alphas: np.ndarray) -> np.ndarray:
    """D[j, t] = prod_{j < i <= t} alpha_i for j <= t (1 on the diagonal), else 0."""
    c = len(alphas)
    D = np.zeros((c, c))
    for t in range(c):
        acc = 1.0
        for j in range(t, -1, -1):
            D[j, t] = acc
            acc *= alphas[j]
    return D


def gamma(alphas: np.ndarray) -> np.ndarray:
    """G[t] = prod_{i <= t} alpha_i."""
    return np.cumprod(alphas)


def m2_replay_output(S0, recs: List[dict], q) -> np.ndarray:
    a = _alphas(recs)
    t = len(recs) - 1
    D = decay_matrix(a)
    y = gamma(a)[t] * (S0 @ q)
    for j, r in enumerate(recs):
        y = y + D[j, t] * (r["k"] @ q) * r["v"]
    return y


def m2_fold(S0, recs: List[dict]) -> np.ndarray:
    a = _alphas(recs)
    t = len(recs) - 1
    D = decay_matrix(a)
    S = gamma(a)[t] * S0
    for j, r in enumerate(recs):
        S = S + D[j, t] * np.outer(r["v"], r["k"])
    return S


def chunk_verify(S0, committed: List[dict], drafts: List[dict], q_drafts, kind: str):
    """O [T, P] = S_0 Q D + U (W o K^T Q) over the chunk committed + drafts."""
    recs = list(committed) + list(drafts)
    h, T = len(committed), len(drafts)
    a = _alphas(recs)
    Dm = decay_matrix(a)
    G = gamma(a)
    K = np.stack([r["k"] for r in recs], axis=1)            # N x c
    Q = np.stack(q_drafts, axis=1)                           # N x T
    cols = [h + tau for tau in range(T)]
    Dd = np.diag(G[cols])
    W = Dm[:, cols]                                          # c x T, zero above the draft
    U = pseudo_values(S0, recs) if kind == "gdn" else np.stack([r["v"] for r in recs], axis=1)
    O = S0 @ Q @ Dd + U @ (W * (K.T @ Q))
    return O.T


def pseudo_values(S0, recs: List[dict]) -> np.ndarray:
    """U (P x c) from the unit lower-triangular solve of the delta rule."""
    a = _alphas(recs)
    b = np.array([r["beta"] for r in recs], np.float64)
    c = len(recs)
    Dm = decay_matrix(a)
    G = gamma(a)
    K = np.stack([r["k"] for r in recs], axis=1)
    V = np.stack([r["v"] for r in recs], axis=1)
    rhs = (V - (S0 @ K) * G[None, :]) * b[None, :]
    A = np.zeros((c, c))                                     # strictly upper: A[i, j], i < j
    KK = K.T @ K
    for j in range(c):
        for i in range(j):
            A[i, j] = b[j] * Dm[i, j] * KK[i, j]
    # U (I + A) = rhs  ->  forward substitution over columns
    U = np.zeros_like(rhs)
    for j in range(c):
        U[:, j] = rhs[:, j] - U[:, :j] @ A[:j, j]
    return U


def gdn_fold(S0, recs: List[dict]) -> np.ndarray:
    a = _alphas(recs)
    t = len(recs) - 1
    Dm = decay_matrix(a)
    U = pseudo_values(S0, recs)
    S = gamma(a)[t] * S0
    for j, r in enumerate(recs):
        S = S + Dm[j, t] * np.outer(U[:, j], r["k"])
    return S


def query_transform_output(S0, recs: List[dict], q, kind: str) -> np.ndarray:
    a = _alphas(recs)
    t = len(recs) - 1
    Dm = decay_matrix(a)
    r = np.array(q, np.float64)
    acc = np.zeros(S0.shape[0])
    for i in range(t, -1, -1):
        c = recs[i]["k"] @ r
        if kind == "gdn":
            bi = recs[i]["beta"]
            acc = acc + Dm[i, t] * bi * c * recs[i]["v"]
            r = r - bi * c * recs[i]["k"]
        else:
            acc = acc + Dm[i, t] * c * recs[i]["v"]
    return acc + gamma(a)[t] * (S0 @ r)


def kda_query_transform_output(S0, recs: List[dict], q) -> np.ndarray:
    """KDA output over the window ``recs`` (``alpha`` an [N] vector per record)."""
    r = np.array(q, np.float64)
    acc = np.zeros(S0.shape[0])
    for rec in reversed(recs):
        c = rec["beta"] * (rec["k"] @ r)
        acc = acc + c * rec["v"]
        r = np.asarray(rec["alpha"], np.float64) * (r - c * rec["k"])
    return acc + S0 @ r
