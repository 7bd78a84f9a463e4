"""Mamba-2 single-token decode, float64.  Test infrastructure only.

Definition (Mamba-2 SSD decode, one token; per sequence and head h, with the
B/C group g = h // (H // G), i.e. contiguous blocks of heads share a group):

    a    = exp(dt_h * A_h)
    S_h <- a * S_h + dt_h * x_h B_g^T            S_h is P x N
    y_h  = S_h C_g + D_h * x_h

The output is read from the state *after* this token's update: the pages
describe the conventional step as load, update, output from the updated
state, store [P3, Interpretation 1].  Reading of silent points: no z-gate, no
causal conv, no dt bias; dt arrives already positive, and the D*x skip is
included.

Replay form (the method: a checkpoint plus a buffer of recent inputs
[P1, Synopsis; P2, paragraph 3; P3, Interpretation 2]).  Let S0 be the
checkpoint and records 1..m the inputs buffered since it, and let
s_j = dt_1 + ... + dt_j.  Unrolling the update m times gives

    S_m = exp(A s_m) S0 + sum_{j<=m} exp(A (s_m - s_j)) dt_j x_j B_j^T

so the newest output needs one read of S0 and the buffered records:

    y_m = exp(A s_m) (S0 C_m) + sum_{j<=m} exp(A (s_m - s_j)) dt_j (B_j . C_m) x_j
          + D x_m

Decay factors are always formed from segment sums s_m - s_j, never as a ratio
of two cumulative decays, which would underflow to 0/0 for strongly decaying
heads.

Decay skip (optional).  A future direction on the pages [P3, Perspective,
paragraph 1]: once a head has decayed so far that the checkpoint no longer
matters, its steps need not load the checkpoint, and its fold only stores
the folded records.  No threshold is given.  Reading taken: the checkpoint
term of a head is dropped when
A s_m < ln 2^-24 (the decay exp(A s_m) is below float32's unit roundoff), in
outputs and in folds alike: replay_output and fold take skip_below = that
logarithm.
"""
from __future__ import annotations

import numpy as np


def head_group(heads: int, groups: int) -> np.ndarray:
    """Group index of every head: contiguous blocks of heads // groups heads."""
    if groups <= 0 or heads % groups:
        raise ValueError("heads must be a multiple of groups")
    return np.arange(heads) // (heads // groups)


def step(S, x, B, C, dt, A, D):
    """One conventional decode step for every (sequence, head).

    S [..., H, P, N]; x [..., H, P]; B, C [..., G, N]; dt [..., H]; A, D [H].
    Returns (S_new, y): the updated state and y [..., H, P] read from it.
    Inputs are not modified.
    """
    S = np.asarray(S, np.float64)
    H, G = x.shape[-2], B.shape[-2]
    g = head_group(H, G)
    Bh = np.asarray(B, np.float64)[..., g, :]          # [..., H, N]
    Ch = np.asarray(C, np.float64)[..., g, :]
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    D = np.asarray(D, np.float64)
    decay = np.exp(dt * A)                              # [..., H]
    outer = (dt[..., None] * x)[..., :, None] * Bh[..., None, :]
    S_new = decay[..., None, None] * S + outer
    y = np.einsum("...pn,...n->...p", S_new, Ch) + D[:, None] * x
    return S_new, y


def _cumsum_dt(recs):
    return np.cumsum(np.stack([np.asarray(r["dt"], np.float64) for r in recs]), axis=0)  # [m, H]


DECAY_SKIP_LOG = -24.0 * np.log(2.0)  # ln 2^-24


def _s0_weight(A, s_m, skip_below):
    """exp(A s_m), or 0 for heads whose decay is below the skip threshold."""
    w = np.exp(A * s_m)
    return w if skip_below is None else np.where(A * s_m < skip_below, 0.0, w)


def replay_output(S0, recs, A, D, skip_below=None):
    """Output of the newest record, from checkpoint S0 and the buffered records.

    One sequence.  S0 [H, P, N]; recs: records 1..m since the checkpoint,
    oldest first, each a dict of x [H, P], B [G, N], C [G, N], dt [H].
    """
    S0 = np.asarray(S0, np.float64)
    A = np.asarray(A, np.float64)
    H, G = S0.shape[0], recs[0]["B"].shape[0]
    g = head_group(H, G)
    s = _cumsum_dt(recs)
    newest = recs[-1]
    Cm = np.asarray(newest["C"], np.float64)[g]          # [H, N]
    y = _s0_weight(A, s[-1], skip_below)[:, None] * np.einsum("hpn,hn->hp", S0, Cm)
    for j, r in enumerate(recs):
        seg = s[-1] - s[j]                              # dt summed over records j+1..m
        Bj = np.asarray(r["B"], np.float64)[g]
        w = np.exp(A * seg) * np.asarray(r["dt"], np.float64) * np.einsum("hn,hn->h", Bj, Cm)
        y = y + w[:, None] * np.asarray(r["x"], np.float64)
    return y + np.asarray(D, np.float64)[:, None] * np.asarray(newest["x"], np.float64)


def fold(S0, recs, A, skip_below=None):
    """New checkpoint after folding records 1..m into S0 (one sequence)."""
    S0 = np.asarray(S0, np.float64)
    A = np.asarray(A, np.float64)
    if not recs:
        return S0.copy()
    H, G = S0.shape[0], recs[0]["B"].shape[0]
    g = head_group(H, G)
    s = _cumsum_dt(recs)
    S = _s0_weight(A, s[-1], skip_below)[:, None, None] * S0
    for j, r in enumerate(recs):
        coef = np.exp(A * (s[-1] - s[j])) * np.asarray(r["dt"], np.float64)          # [H]
        xj = np.asarray(r["x"], np.float64)
        Bj = np.asarray(r["B"], np.float64)[g]
        S = S + coef[:, None, None] * xj[:, :, None] * Bj[:, None, :]
    return S


def output_scale(S, C, D, x):
    """Size of the terms an output sums, per head: max_p (|S| |C|)_p + |D| max_p |x_p|.

    One sequence after a token: S [H, P, N] the state the output reads, C [G, N],
    x [H, P].  A relative error of a head's output vector is measured against
    the larger of this and the output itself (a head's output can cancel).
    """
    S = np.abs(np.asarray(S, np.float64))
    H, G = S.shape[0], np.shape(C)[0]
    Ch = np.abs(np.asarray(C, np.float64))[head_group(H, G)]
    return (np.einsum("hpn,hn->hp", S, Ch).max(axis=-1)
            + np.abs(np.asarray(D, np.float64)) * np.abs(np.asarray(x, np.float64)).max(axis=-1))
