"""Stepwise fp64 recurrences (oracle; test infrastructure only).

One call advances every head of one sequence by one record.  Shapes:
S [H, P, N] (float64), alpha/beta [H], v [H, P], k/q [G, N]; value head h reads
key/query head h // (H // G).

Mamba-2 -- page 4 "What shipped": S_t = a_t S_{t-1} + v_t k_t^T.  The output is
read from the post-update state, y_t = S_t q_t (the usual Mamba-2 readout with
q in the role of C; the pages give only the update).

Gated DeltaNet -- the pages name the gated delta-rule update (page 1, models
section; page 4, "What shipped" and "Why it matters") without a formula.  The
reading used here is the published Gated DeltaNet rule
    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
evaluated in the order: decay, error against the decayed state, rank-1 write.

Kimi Delta Attention (KDA) -- page 1 (models section) and page 4 (opening
paragraph) list KDA as the SSM layer of Kimi-K3; page 4 "Why it matters" says
the replay reframing carries over to KDA's delta-rule update, and page 4
"Caveats" notes KDA was not evaluated.  No formula is given.  The reading used
here is KDA's own publication (Kimi Linear): Gated DeltaNet with the scalar gate
replaced by a per-key-channel gate a_t in (0, 1]^N,
    S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
in this [P][N] orientation (rows: value dim, columns: key dim), again evaluated
as decay, error against the decayed state, rank-1 write.  The gate is per value
head: alpha has shape [H, N].

Parity unpinned: that the Gated DeltaNet and KDA forms above are the ones the
pages' own kernels compute (the pages give neither formula).  The oracle's
evaluation of these forms is pinned (tests/test_oracle_pins.py,
tests/test_oracle_kda.py: Kronecker unrolling, exact rationals, special cases).
"""
from __future__ import annotations

import numpy as np


def widen(x, in_dtype: str) -> np.ndarray:
    """Exact widening of stored inputs to float64 (bf16 arrays hold raw bits)."""
    x = np.asarray(x)
    if in_dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 inputs are uint16 bit patterns")
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if in_dtype == "fp32":
        if x.dtype != np.float32:
            raise TypeError("fp32 inputs are float32 arrays")
        return x.astype(np.float64)
    raise ValueError(in_dtype)


def expand_heads(x: np.ndarray, n_heads: int) -> np.ndarray:
    """[G, N] key/query rows -> [H, N] with value head h using row h // (H // G)."""
    G = x.shape[0]
    if n_heads % G:
        raise ValueError("H must be a multiple of G")
    return np.repeat(x, n_heads // G, axis=0)


def mamba2_step(S, alpha, v, k, q):
    """S <- alpha S + v k^T ; y = S q.  Returns (S_new, y)."""
    H = S.shape[0]
    kh = expand_heads(k, H)
    qh = expand_heads(q, H)
    S_new = alpha[:, None, None] * S + v[:, :, None] * kh[:, None, :]
    y = np.einsum("hpn,hn->hp", S_new, qh)
    return S_new, y


def gdn_step(S, alpha, beta, v, k, q):
    """S <- alpha S ; u = beta (v - S k) ; S <- S + u k^T ; o = S q."""
    H = S.shape[0]
    kh = expand_heads(k, H)
    qh = expand_heads(q, H)
    Sd = alpha[:, None, None] * S
    u = beta[:, None] * (v - np.einsum("hpn,hn->hp", Sd, kh))
    S_new = Sd + u[:, :, None] * kh[:, None, :]
    o = np.einsum("hpn,hn->hp", S_new, qh)
    return S_new, o


def kda_step(S, alpha, beta, v, k, q):
    """S <- S Diag(alpha_h) ; u = beta (v - S k) ; S <- S + u k^T ; o = S q.  alpha [H, N]."""
    H = S.shape[0]
    kh = expand_heads(k, H)
    qh = expand_heads(q, H)
    Sd = S * alpha[:, None, :]
    u = beta[:, None] * (v - np.einsum("hpn,hn->hp", Sd, kh))
    S_new = Sd + u[:, :, None] * kh[:, None, :]
    o = np.einsum("hpn,hn->hp", S_new, qh)
    return S_new, o


def step(kind: str, S, rec):
    """Advance by one record ``rec`` = dict(alpha, beta, v, k, q) of float64 arrays."""
    if kind == "mamba2":
        return mamba2_step(S, rec["alpha"], rec["v"], rec["k"], rec["q"])
    if kind == "gdn":
        return gdn_step(S, rec["alpha"], rec["beta"], rec["v"], rec["k"], rec["q"])
    if kind == "kda":
        return kda_step(S, rec["alpha"], rec["beta"], rec["v"], rec["k"], rec["q"])
    raise ValueError(kind)
