"""The replay session (the method) against the stepwise session (the definition),
through the whole call surface: step, verify, commit, flush."""
import numpy as np
import pytest

from oracle.session import ReplaySession, StepwiseSession
from synth import InputStream, LayerShape


def _shape(kind, L):
    if kind == "mamba2":
        return LayerShape("mamba2", 4, 4, 3, 5, 2, L)
    return LayerShape("gdn", 4, 3, 5, 6, 3, L)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("L", [1, 4, 6])
def test_speculative_calls_match_definition(kind, L):
    s = _shape(kind, L)
    ins = InputStream(s, seed=L)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    ref = StepwiseSession(kind, S0, ins.params)
    rep = ReplaySession(kind, S0, L, ins.params)
    rng = np.random.default_rng(100 + L)
    for it in range(40):
        op = rng.integers(3)
        if op == 0:
            r = ins.record()
            np.testing.assert_allclose(rep.step(r), ref.step(r), rtol=1e-9, atol=1e-11)
        elif op == 1:
            T = int(rng.integers(1, L + 1))
            d = ins.drafts(T)
            np.testing.assert_allclose(rep.verify(d), ref.verify(d), rtol=1e-9, atol=1e-11)
            a = ins.accepted(T)
            rep.commit(a)
            ref.commit(a)
        else:
            mask = rng.integers(0, 2, size=s.batch).astype(bool)
            folded = rep.flush(mask)
            ref.flush(mask)
            for b in np.nonzero(folded)[0]:
                # After an explicit flush the checkpoint is the exact state.
                np.testing.assert_allclose(rep.ckpt[b], ref.state[b], rtol=1e-9, atol=1e-11)
    rep.flush()
    np.testing.assert_allclose(rep.ckpt, ref.state, rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_verify_without_fold_leaves_checkpoint(kind):
    s = _shape(kind, 8)
    ins = InputStream(s, seed=3)
    rep = ReplaySession(kind, ins.initial_state(zeros=False), 8, ins.params)
    for _ in range(3):
        rep.step(ins.record())
    before = rep.ckpt.copy()
    rep.verify(ins.drafts(4))                            # 3 + 4 <= 8: no fold
    np.testing.assert_array_equal(rep.ckpt, before)
    rep.commit(np.zeros(s.batch, np.int32))
    np.testing.assert_array_equal(rep.ckpt, before)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_commit_then_continue_equals_stepping_accepted(kind):
    # Accepting a drafts and continuing equals stepping those a tokens directly.
    s = _shape(kind, 5)
    ins = InputStream(s, seed=9)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    r0, d, r1 = ins.record(), ins.drafts(4), ins.record()
    a = np.array([0, 1, 3, 4], np.int32)
    rep = ReplaySession(kind, S0, 5, ins.params)
    rep.step(r0)
    rep.verify(d)
    rep.commit(a)
    y_rep = rep.step(r1)
    ref = StepwiseSession(kind, S0, ins.params)
    ref.step(r0)
    for b in range(s.batch):
        for i in range(a[b]):
            ref.state[b], _ = ref.k.step(ref.state[b], {n: x[b, i] for n, x in d.items()})
    np.testing.assert_allclose(y_rep, ref.step(r1), rtol=1e-9, atol=1e-11)
    assert list(rep.ptr.pos) == [2, 3, 5, 6]


def test_output_scale_bounds_the_output():
    """The output scale is the sum of the terms' magnitudes: it bounds |y| for any
    signs (triangle inequality) and equals it when every term is non-negative."""
    from oracle import gdn, mamba2
    rng = np.random.default_rng(2)
    H, G, P, N = 4, 2, 8, 16
    S, C, x = rng.standard_normal((H, P, N)), rng.standard_normal((G, N)), rng.standard_normal((H, P))
    D = rng.standard_normal(H)
    g = mamba2.head_group(H, G)
    y = np.einsum("hpn,hn->hp", S, C[g]) + D[:, None] * x
    assert np.all(mamba2.output_scale(S, C, D, x) >= np.abs(y).max(-1) - 1e-12)
    Sp, Cp, xp, Dp = np.abs(S), np.abs(C), np.abs(x), np.abs(D)
    yp = np.einsum("hpn,hn->hp", Sp, Cp[g]) + Dp[:, None] * xp
    # equal when the largest row of |S||C| also holds the largest |x| (make x constant per head)
    xc = np.ones_like(xp)
    yc = np.einsum("hpn,hn->hp", Sp, Cp[g]) + Dp[:, None] * xc
    np.testing.assert_allclose(mamba2.output_scale(Sp, Cp, Dp, xc), yc.max(-1), rtol=1e-14)
    assert np.all(mamba2.output_scale(Sp, Cp, Dp, xp) >= yp.max(-1) - 1e-12)
    Sg, q = rng.standard_normal((H, P, N)), rng.standard_normal((H, N))
    o = np.einsum("hvk,hk->hv", Sg, q)
    assert np.all(gdn.output_scale(Sg, q) >= np.abs(o).max(-1) - 1e-12)
    np.testing.assert_allclose(gdn.output_scale(np.abs(Sg), np.abs(q)),
                               np.einsum("hvk,hk->hv", np.abs(Sg), np.abs(q)).max(-1), rtol=1e-14)
