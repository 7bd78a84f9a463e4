"""Pins for the Gated DeltaNet oracle: closed forms, delta-rule identities,
explicit-matrix brute force and the UT/WY replay identity."""
import numpy as np
import pytest

from oracle import gdn
from oracle.session import ReplaySession, StepwiseSession


def _unit(v):
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _rec(rng, H, dk, dv, lead=()):
    return {"q": _unit(rng.standard_normal(lead + (H, dk))), "k": _unit(rng.standard_normal(lead + (H, dk))),
            "v": rng.standard_normal(lead + (H, dv)),
            "alpha": np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal(lead + (H,))))),
            "beta": 1 / (1 + np.exp(-rng.standard_normal(lead + (H,))))}


def test_one_step_from_zero_state():
    # S0 = 0: S = beta v k^T and o = beta (k.q) v.
    rng = np.random.default_rng(1)
    H, dk, dv = 2, 5, 3
    r = _rec(rng, H, dk, dv)
    S, o = gdn.step(np.zeros((H, dv, dk)), r["q"], r["k"], r["v"], r["alpha"], r["beta"])
    for h in range(H):
        kq = sum(r["k"][h, i] * r["q"][h, i] for i in range(dk))
        for i in range(dv):
            assert abs(o[h, i] - r["beta"][h] * kq * r["v"][h, i]) < 1e-12


def test_delta_rule_writes_value_at_key():
    # alpha = beta = 1 and a unit key: the update makes S k = v exactly.
    rng = np.random.default_rng(2)
    H, dk, dv = 3, 6, 4
    S0 = rng.standard_normal((H, dv, dk))
    r = _rec(rng, H, dk, dv)
    S, _ = gdn.step(S0, r["q"], r["k"], r["v"], np.ones(H), np.ones(H))
    np.testing.assert_allclose(np.einsum("hvk,hk->hv", S, r["k"]), r["v"], rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_are_independent_slots():
    # alpha = beta = 1, keys e_0..e_3 written in turn: S e_i = v_i for every i.
    H, dk, dv = 1, 4, 3
    rng = np.random.default_rng(3)
    S = np.zeros((H, dv, dk))
    vs = rng.standard_normal((dk, H, dv))
    for i in range(dk):
        e = np.zeros((H, dk)); e[:, i] = 1.0
        S, o = gdn.step(S, e, e, vs[i], np.ones(H), np.ones(H))
        np.testing.assert_array_equal(o, vs[i])
    for i in range(dk):
        np.testing.assert_array_equal(S[:, :, i], vs[i])


def test_alpha_one_beta_zero_is_identity():
    rng = np.random.default_rng(4)
    H, dk, dv = 2, 5, 3
    S0 = rng.standard_normal((H, dv, dk))
    r = _rec(rng, H, dk, dv)
    S, o = gdn.step(S0, r["q"], r["k"], r["v"], np.ones(H), np.zeros(H))
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("hvk,hk->hv", S0, r["q"]), rtol=1e-13)


def test_beta_zero_is_pure_decay():
    # beta = 0: S_m = (alpha_1 ... alpha_m) S0 and o_m = exp(sum log alpha) S0 q_m.
    rng = np.random.default_rng(5)
    H, dk, dv = 2, 4, 3
    S0 = rng.standard_normal((H, dv, dk))
    recs = [_rec(rng, H, dk, dv) for _ in range(5)]
    for r in recs:
        r["beta"] = np.zeros(H)
    S = S0.copy()
    prod = np.ones(H)
    for t, r in enumerate(recs):
        S, o = gdn.step(S, r["q"], r["k"], r["v"], r["alpha"], r["beta"])
        prod = prod * r["alpha"]
        np.testing.assert_allclose(o, prod[:, None] * np.einsum("hvk,hk->hv", S0, r["q"]), rtol=1e-12)
        np.testing.assert_allclose(gdn.replay_output(S0, recs[:t + 1], r["q"]), o, rtol=1e-12)


def test_stepwise_matches_explicit_matrix_update():
    # Brute force: form alpha (I - beta k k^T) as a dk x dk matrix and multiply.
    rng = np.random.default_rng(6)
    H, dk, dv = 2, 5, 4
    S = rng.standard_normal((H, dv, dk))
    Sb = S.copy()
    for _ in range(6):
        r = _rec(rng, H, dk, dv)
        S, o = gdn.step(S, r["q"], r["k"], r["v"], r["alpha"], r["beta"])
        for h in range(H):
            k = r["k"][h][:, None]
            M = r["alpha"][h] * (np.eye(dk) - r["beta"][h] * (k @ k.T))
            Sb[h] = Sb[h] @ M + r["beta"][h] * (r["v"][h][:, None] @ k.T)
            np.testing.assert_allclose(o[h], Sb[h] @ r["q"][h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S, Sb, rtol=1e-11, atol=1e-12)


def test_pseudo_values_match_definition():
    # u_t = beta_t (v_t - alpha_t S_{t-1} k_t), with S_{t-1} from the stepwise state.
    rng = np.random.default_rng(7)
    H, dk, dv, m = 3, 6, 4, 7
    S0 = rng.standard_normal((H, dv, dk))
    recs = [_rec(rng, H, dk, dv) for _ in range(m)]
    U = gdn.pseudo_values(S0, recs)
    S = S0.copy()
    for t, r in enumerate(recs):
        u_def = r["beta"][:, None] * (r["v"] - r["alpha"][:, None] * np.einsum("hvk,hk->hv", S, r["k"]))
        np.testing.assert_allclose(U[t], u_def, rtol=1e-11, atol=1e-12)
        S, _ = gdn.step(S, r["q"], r["k"], r["v"], r["alpha"], r["beta"])
    np.testing.assert_allclose(gdn.fold(S0, recs), S, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("L", [1, 3, 16])
def test_replay_session_equals_stepwise(L):
    rng = np.random.default_rng(20 + L)
    Bt, H, dk, dv = 2, 3, 6, 5
    S0 = rng.standard_normal((Bt, H, dv, dk))
    ref = StepwiseSession("gdn", S0)
    rep = ReplaySession("gdn", S0, L)
    for t in range(3 * L + 4):
        r = _rec(rng, H, dk, dv, (Bt,))
        state_before = ref.state.copy()
        np.testing.assert_allclose(rep.step(r), ref.step(r), rtol=1e-10, atol=1e-12)
        if L == 1 and t > 0:
            np.testing.assert_allclose(rep.ckpt, state_before, rtol=1e-12, atol=1e-12)


def test_decay_skip_drops_exactly_the_checkpoint_term():
    """With the decay skip, a head whose window log-decay g_m is below ln 2^-24
    gives exactly the output (and fold) of a zero checkpoint, every other head
    exactly the full replay form, and the skipped term moves the output by at
    most 2^-24 ||S0||_2 ||q||: S0 enters only through exp(g_m) S0 times a product
    of I - beta k k^T, each of norm <= 1 [P3, Perspective, paragraph 1]."""
    from oracle.mamba2 import DECAY_SKIP_LOG as thr
    rng = np.random.default_rng(12)
    H, dv, dk, m = 4, 6, 8, 9
    S0 = rng.standard_normal((H, dv, dk))
    log_alpha = np.array([-30.0, -0.01, -2.5, -0.5])     # per record
    recs = []
    for _ in range(m):
        k = rng.standard_normal((H, dk))
        q = rng.standard_normal((H, dk))
        recs.append({"k": k / np.linalg.norm(k, axis=-1, keepdims=True),
                     "q": q / np.linalg.norm(q, axis=-1, keepdims=True),
                     "v": rng.standard_normal((H, dv)), "beta": rng.uniform(0.1, 0.9, H),
                     "alpha": np.exp(log_alpha * rng.uniform(0.8, 1.2, H))})
    zero = np.zeros_like(S0)
    for n in range(1, m + 1):
        w = recs[:n]
        g = np.sum([np.log(r["alpha"]) for r in w], axis=0)
        skipped = g < thr
        q = w[-1]["q"]
        y_skip, y_full, y_zero = (gdn.replay_output(S, w, q, skip_below=sk)
                                  for S, sk in ((S0, thr), (S0, None), (zero, None)))
        f_skip, f_full, f_zero = (gdn.fold(S, w, skip_below=sk) for S, sk in ((S0, thr), (S0, None), (zero, None)))
        for h in range(H):
            want_y, want_f = (y_zero[h], f_zero[h]) if skipped[h] else (y_full[h], f_full[h])
            np.testing.assert_allclose(y_skip[h], want_y, rtol=0, atol=1e-12)
            np.testing.assert_allclose(f_skip[h], want_f, rtol=0, atol=1e-12)
            if skipped[h]:
                bound = 2.0 ** -24 * np.linalg.norm(S0[h], 2) * np.linalg.norm(q[h])
                assert np.linalg.norm(y_skip[h] - y_full[h]) <= bound * (1 + 1e-9)
    g_all = np.cumsum([np.log(r["alpha"]) for r in recs], axis=0)
    assert g_all[0, 0] < thr and g_all[-1, 1] > thr and g_all[0, 2] > thr > g_all[-1, 2]
