"""Gated DeltaNet single-token decode, float64.  Test infrastructure only.

Definition (Gated DeltaNet decode, one token; per sequence and head; the state
S is d_v x d_k, applied to keys from the right):

    S <- alpha * S (I - beta k k^T) + beta v k^T
    o  = S q

with no 1/sqrt(d_k) scaling of q (reading of a silent point).  Written out,
the update is S <- alpha S + u k^T with the pseudo-value

    u = beta (v - alpha S k).

Replay form (checkpoint plus buffered records [P1, Synopsis; P3,
Interpretation 2]).  Let S0 be the checkpoint, records 1..m the inputs since
it, and g_j = log alpha_1 + ... + log alpha_j.  Unrolling the update gives

    S_m = exp(g_m) S0 + sum_{j<=m} exp(g_m - g_j) u_j k_j^T              (fold)

and substituting S_{t-1} into u_t gives, for every t <= m,

    u_t + beta_t sum_{j<t} exp(g_t - g_j) (k_t . k_j) u_j
        = beta_t (v_t - exp(g_t) S0 k_t)

i.e. a unit-lower-triangular system (I + Acal) U = diag(beta)(V - diag(e^g) K S0^T)
in the pseudo-values (the UT / WY form), solved by forward substitution.  The
newest output is then

    o_m = exp(g_m) S0 q_m + sum_{j<=m} exp(g_m - g_j) (k_j . q_m) u_j.

Only S0 k_j (j <= m) and S0 q_m touch the checkpoint, so one read of S0
serves the whole window.

Decay skip (optional; the pages' future direction for heads whose decay has
made the checkpoint irrelevant [P3, Perspective, paragraph 1], with no
threshold given).  Every way the checkpoint enters the newest output or the
fold carries the factor exp(g_m): S_m = exp(g_m) S0 prod_t (I - beta_t k_t
k_t^T) + (terms without S0), and each factor I - beta k k^T has norm at most 1
for unit keys and 0 <= beta <= 2.  Reading taken, as for Mamba-2: when
g_m < ln 2^-24 the computation (its pseudo-values and output, or the fold)
uses a zero checkpoint, which moves an output by at most 2^-24 |S0| |q|.
"""
from __future__ import annotations

import numpy as np


def step(S, q, k, v, alpha, beta):
    """One conventional decode step for every (sequence, head).

    S [..., H, dv, dk]; q, k [..., H, dk]; v [..., H, dv]; alpha, beta [..., H].
    Returns (S_new, o) with o [..., H, dv] read from S_new.
    """
    S = np.asarray(S, np.float64)
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    a = np.asarray(alpha, np.float64)[..., None, None]
    b = np.asarray(beta, np.float64)[..., None, None]
    Sk = np.einsum("...vk,...k->...v", S, k)
    S_new = a * (S - b * Sk[..., :, None] * k[..., None, :]) + b * v[..., :, None] * k[..., None, :]
    o = np.einsum("...vk,...k->...v", S_new, q)
    return S_new, o


def _log_decay_cumsum(recs):
    return np.cumsum(np.stack([np.log(np.asarray(r["alpha"], np.float64)) for r in recs]), axis=0)  # [m, H]


def pseudo_values(S0, recs):
    """U [m, H, dv]: forward substitution of the window's triangular system.

    One sequence.  S0 [H, dv, dk]; recs: records 1..m since the checkpoint,
    oldest first, each a dict of k [H, dk], v [H, dv], alpha [H], beta [H].
    """
    S0 = np.asarray(S0, np.float64)
    g = _log_decay_cumsum(recs)
    K = [np.asarray(r["k"], np.float64) for r in recs]
    U = []
    for t, r in enumerate(recs):
        beta_t = np.asarray(r["beta"], np.float64)
        rhs = beta_t[:, None] * (np.asarray(r["v"], np.float64)
                                 - np.exp(g[t])[:, None] * np.einsum("hvk,hk->hv", S0, K[t]))
        for j in range(t):
            coupling = beta_t * np.exp(g[t] - g[j]) * np.einsum("hk,hk->h", K[t], K[j])
            rhs = rhs - coupling[:, None] * U[j]
        U.append(rhs)
    return np.stack(U)


def _skip_checkpoint(S0, g_last, skip_below):
    """S0 with the heads whose window log-decay is below skip_below zeroed."""
    if skip_below is None:
        return S0
    return np.where((g_last < skip_below)[:, None, None], 0.0, S0)


def replay_output(S0, recs, q, skip_below=None):
    """Output for the newest record (query q [H, dk]) from S0 and the window."""
    S0 = np.asarray(S0, np.float64)
    q = np.asarray(q, np.float64)
    g = _log_decay_cumsum(recs)
    S0 = _skip_checkpoint(S0, g[-1], skip_below)
    U = pseudo_values(S0, recs)
    o = np.exp(g[-1])[:, None] * np.einsum("hvk,hk->hv", S0, q)
    for j, r in enumerate(recs):
        kq = np.einsum("hk,hk->h", np.asarray(r["k"], np.float64), q)
        o = o + (np.exp(g[-1] - g[j]) * kq)[:, None] * U[j]
    return o


def fold(S0, recs, skip_below=None):
    """New checkpoint after folding records 1..m into S0 (one sequence)."""
    S0 = np.asarray(S0, np.float64)
    if not recs:
        return S0.copy()
    g = _log_decay_cumsum(recs)
    S0 = _skip_checkpoint(S0, g[-1], skip_below)
    U = pseudo_values(S0, recs)
    S = np.exp(g[-1])[:, None, None] * S0
    for j, r in enumerate(recs):
        kj = np.asarray(r["k"], np.float64)
        S = S + np.exp(g[-1] - g[j])[:, None, None] * U[j][:, :, None] * kj[:, None, :]
    return S


def output_scale(S, q):
    """Size of the terms an output sums, per head: max_v (|S| |q|)_v.

    One sequence after a token: S [H, dv, dk] the state the output reads,
    q [H, dk].  See mamba2.output_scale.
    """
    return np.einsum("hvk,hk->hv", np.abs(np.asarray(S, np.float64)),
                     np.abs(np.asarray(q, np.float64))).max(axis=-1)
