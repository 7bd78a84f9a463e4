"""Pins for the Mamba-2 oracle: closed forms, brute force and the replay identity.

Each test checks the oracle against something it does not compute itself: a
closed form of the recurrence, an explicit-product unrolling written with
plain loops, or the other of its two formulations (stepwise vs replay).
"""
import numpy as np
import pytest

from oracle import mamba2
from oracle.session import ReplaySession, StepwiseSession


def _rand_layer(rng, H=3, P=5, N=4, G=1):
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    return A, D


def _rec(rng, H, P, N, G, lead=()):
    return {"x": rng.standard_normal(lead + (H, P)), "B": rng.standard_normal(lead + (G, N)),
            "C": rng.standard_normal(lead + (G, N)),
            "dt": np.log1p(np.exp(rng.standard_normal(lead + (H,)) - 2))}


def test_one_step_from_zero_state():
    # From S0 = 0 a single token gives S = dt x B^T, so y = dt (B.C) x + D x.
    rng = np.random.default_rng(1)
    H, P, N = 3, 5, 4
    A, D = _rand_layer(rng, H, P, N)
    r = _rec(rng, H, P, N, 1)
    S, y = mamba2.step(np.zeros((H, P, N)), r["x"], r["B"], r["C"], r["dt"], A, D)
    for h in range(H):
        bc = sum(r["B"][0, n] * r["C"][0, n] for n in range(N))
        for p in range(P):
            expect = r["dt"][h] * bc * r["x"][h, p] + D[h] * r["x"][h, p]
            assert abs(y[h, p] - expect) < 1e-12
            for n in range(N):
                assert abs(S[h, p, n] - r["dt"][h] * r["x"][h, p] * r["B"][0, n]) < 1e-12


def test_constant_input_geometric_series():
    # Repeating one record t times from S0 = 0: S_t = dt x B^T (1 - a^t) / (1 - a), a = exp(dt A).
    rng = np.random.default_rng(2)
    H, P, N = 2, 3, 4
    A, D = _rand_layer(rng, H, P, N)
    r = _rec(rng, H, P, N, 1)
    S = np.zeros((H, P, N))
    for t in range(1, 12):
        S, y = mamba2.step(S, r["x"], r["B"], r["C"], r["dt"], A, D)
        a = np.exp(r["dt"] * A)
        geo = (1 - a ** t) / (1 - a)
        bc = float(r["B"][0] @ r["C"][0])
        expect = (r["dt"] * geo * bc)[:, None] * r["x"] + D[:, None] * r["x"]
        np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_zero_dt_leaves_state_and_reads_it():
    # dt = 0: decay 1 and no input term, so S is unchanged and y = S0 C + D x.
    rng = np.random.default_rng(3)
    H, P, N = 4, 6, 5
    A, D = _rand_layer(rng, H, P, N)
    S0 = rng.standard_normal((H, P, N))
    r = _rec(rng, H, P, N, 1)
    r["dt"] = np.zeros(H)
    S, y = mamba2.step(S0, r["x"], r["B"], r["C"], r["dt"], A, D)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(y, S0 @ r["C"][0] + D[:, None] * r["x"], rtol=1e-13)


def test_heads_use_contiguous_groups():
    # H=4, G=2: heads 0,1 read group 0 and heads 2,3 read group 1.  One-hot B/C
    # per group make the group visible in the output.
    H, P, N, G = 4, 1, 2, 2
    A = -np.ones(H)
    D = np.zeros(H)
    B = np.array([[1.0, 0.0], [0.0, 1.0]])
    C = np.array([[1.0, 0.0], [0.0, 2.0]])
    x = np.ones((H, P))
    dt = np.full(H, 0.5)
    S, y = mamba2.step(np.zeros((H, P, N)), x, B, C, dt, A, D)
    np.testing.assert_allclose(y[:, 0], [0.5, 0.5, 1.0, 1.0])
    np.testing.assert_allclose(S[:2, 0, 1], 0.0)
    np.testing.assert_allclose(S[2:, 0, 0], 0.0)


def _ssd_unrolled(S0, recs, A, D, g):
    """Brute-force unrolling with explicit products of per-token decays (loops)."""
    T, (H, P, N) = len(recs), S0.shape
    out = np.zeros((T, H, P))
    for t in range(T):
        for h in range(H):
            Ct = recs[t]["C"][g[h]]
            prod_all = 1.0
            for i in range(t + 1):
                prod_all *= np.exp(recs[i]["dt"][h] * A[h])
            for p in range(P):
                acc = prod_all * sum(S0[h, p, n] * Ct[n] for n in range(N))
                for s in range(t + 1):
                    prod = 1.0
                    for i in range(s + 1, t + 1):
                        prod *= np.exp(recs[i]["dt"][h] * A[h])
                    bc = sum(recs[s]["B"][g[h], n] * Ct[n] for n in range(N))
                    acc += bc * prod * recs[s]["dt"][h] * recs[s]["x"][h, p]
                out[t, h, p] = acc + D[h] * recs[t]["x"][h, p]
    return out


def test_stepwise_and_replay_match_bruteforce_unrolling():
    rng = np.random.default_rng(4)
    H, P, N, G, T = 4, 2, 3, 2, 6
    A, D = _rand_layer(rng, H, P, N)
    S0 = rng.standard_normal((H, P, N))
    recs = [_rec(rng, H, P, N, G) for _ in range(T)]
    g = mamba2.head_group(H, G)
    brute = _ssd_unrolled(S0, recs, A, D, g)
    S = S0.copy()
    for t in range(T):
        S, y = mamba2.step(S, recs[t]["x"], recs[t]["B"], recs[t]["C"], recs[t]["dt"], A, D)
        np.testing.assert_allclose(y, brute[t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(mamba2.replay_output(S0, recs[:t + 1], A, D), brute[t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(mamba2.fold(S0, recs, A), S, rtol=1e-11, atol=1e-12)


def test_fold_is_linear_in_checkpoint():
    rng = np.random.default_rng(5)
    H, P, N, G = 2, 3, 4, 1
    A, _ = _rand_layer(rng, H, P, N)
    recs = [_rec(rng, H, P, N, G) for _ in range(5)]
    S0, S1 = rng.standard_normal((2, H, P, N))
    lhs = mamba2.fold(S0 + 2 * S1, recs, A) - mamba2.fold(np.zeros((H, P, N)), recs, A)
    s = sum(r["dt"] for r in recs)
    np.testing.assert_allclose(lhs, np.exp(A * s)[:, None, None] * (S0 + 2 * S1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 4, 16])
def test_replay_session_equals_stepwise(L):
    rng = np.random.default_rng(10 + L)
    Bt, H, P, N, G = 3, 4, 3, 5, 2
    A, D = _rand_layer(rng, H, P, N)
    S0 = rng.standard_normal((Bt, H, P, N))
    ref = StepwiseSession("mamba2", S0, {"A": A, "D": D})
    rep = ReplaySession("mamba2", S0, L, {"A": A, "D": D})
    for t in range(3 * L + 5):
        r = _rec(rng, H, P, N, G, (Bt,))
        state_before = ref.state.copy()
        y_ref = ref.step(r)
        y_rep = rep.step(r)
        np.testing.assert_allclose(y_rep, y_ref, rtol=1e-10, atol=1e-12)
        if L == 1 and t > 0:
            # L = 1 is conventional decoding: every step folds the previous token,
            # so the checkpoint is the full state before this token.
            np.testing.assert_allclose(rep.ckpt, state_before, rtol=1e-12, atol=1e-12)


def test_decay_skip_drops_exactly_the_checkpoint_term():
    """With the decay skip, a head whose window decay A s_m is below ln 2^-24
    gives exactly the output (and fold) of a zero checkpoint, and every other
    head exactly the full replay form; the dropped term is below 2^-24 of
    |S0 C| [P3, Perspective, paragraph 1]."""
    rng = np.random.default_rng(4)
    H, P, N, G, m = 4, 3, 5, 2, 9
    A = np.array([-400.0, -0.01, -20.0, -1.0])
    D = rng.standard_normal(H)
    S0 = rng.standard_normal((H, P, N))
    recs = [{"x": rng.standard_normal((H, P)), "B": rng.standard_normal((G, N)), "C": rng.standard_normal((G, N)),
             "dt": rng.uniform(0.05, 0.3, H)} for _ in range(m)]
    thr = mamba2.DECAY_SKIP_LOG
    assert abs(thr - np.log(2.0 ** -24)) < 1e-12
    zero = np.zeros_like(S0)
    for k in range(1, m + 1):
        window = recs[:k]
        s = np.sum([r["dt"] for r in window], axis=0)
        skipped = A * s < thr
        y_skip = mamba2.replay_output(S0, window, A, D, skip_below=thr)
        y_full = mamba2.replay_output(S0, window, A, D)
        y_zero = mamba2.replay_output(zero, window, A, D)
        f_skip = mamba2.fold(S0, window, A, skip_below=thr)
        f_full, f_zero = mamba2.fold(S0, window, A), mamba2.fold(zero, window, A)
        for h in range(H):
            want_y, want_f = (y_zero[h], f_zero[h]) if skipped[h] else (y_full[h], f_full[h])
            np.testing.assert_allclose(y_skip[h], want_y, rtol=0, atol=1e-12)
            np.testing.assert_allclose(f_skip[h], want_f, rtol=0, atol=1e-12)
            if skipped[h]:
                g = h // (H // G)
                bound = 2.0 ** -24 * np.abs(S0[h] @ window[-1]["C"][g]).max()
                assert np.abs(y_skip[h] - y_full[h]).max() <= bound
    # head 0 skips from the first record on, head 1 never, head 2 from some record within the window
    assert A[0] * recs[0]["dt"][0] < thr and A[1] * np.sum([r["dt"][1] for r in recs]) > thr
    s2 = np.cumsum([r["dt"][2] for r in recs])
    assert A[2] * s2[0] > thr and A[2] * s2[-1] < thr
