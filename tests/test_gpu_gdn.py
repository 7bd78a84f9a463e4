"""Gated DeltaNet replay decode on the GPU against the CPU oracle.

Same bar as the Mamba-2 tests: per-token relative error <= 1e-4 against the
float64 stepwise definition, pointers and status bit-exact against the
oracle's pointer machine, checkpoints after a fold <= 1e-4 of the exact state.
"""
import numpy as np
import pytest

from _gpu import announce, ckpt_rel_err, host, pointers_host, to_dev
from _metrics import max_rel_err
from oracle.pointers import PointerMachine
from oracle.session import ReplaySession, StepwiseSession
from synth import WORKLOADS, InputStream, LayerShape, take_batch

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _layer(shape, max_draft=0, ckpt0=None):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    return ReplayLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       max_draft=max_draft, ckpt0=ckpt0)


def _run_steps(shape, seed, steps, zero_state=True):
    announce("gdn steps", shape, "seed", seed, "steps", steps)
    ins = InputStream(shape, seed)
    S0 = ins.initial_state(zeros=zero_state, scale=0.3)
    lay = _layer(shape, ckpt0=S0)
    ref = StepwiseSession("gdn", S0)
    rep = ReplaySession("gdn", S0, shape.window)
    worst = 0.0
    for t in range(steps):
        r = ins.record()
        y = host(lay.step(to_dev(r)))
        worst = max(worst, max_rel_err(y, ref.step(r), ref.scale))
        rep.step(r)
        pos, ck = pointers_host(lay)
        assert np.array_equal(pos, rep.ptr.pos) and np.array_equal(ck, rep.ptr.ckpt_pos), t
    assert worst <= TOL, worst
    assert ckpt_rel_err(host(lay.checkpoint), rep.ckpt) <= TOL
    assert lay.status == 0


@pytest.mark.parametrize("shape", [
    LayerShape("gdn", 2, 4, 64, 32, 4, 4),         # small, every step
    LayerShape("gdn", 3, 4, 128, 128, 4, 5),       # full head size, odd window, ragged step count
    LayerShape("gdn", 2, 3, 128, 64, 3, 16),       # L = 16, batch*heads not a multiple of 8
    LayerShape("gdn", 1, 5, 64, 128, 5, 1),        # L = 1: conventional decoding
])
def test_shapes(shape):
    _run_steps(shape, seed=7, steps=2 * shape.window + 3, zero_state=False)


def test_zero_initial_state():
    _run_steps(LayerShape("gdn", 2, 2, 64, 64, 2, 6), seed=2, steps=20)


def _spec_run(shape, seed, ops, T_max):
    import torch
    announce("gdn speculative", shape, "seed", seed)
    ins = InputStream(shape, seed)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    lay = _layer(shape, max_draft=T_max, ckpt0=S0)
    ref = StepwiseSession("gdn", S0)
    pm = PointerMachine(shape.batch, shape.window)
    rng = np.random.default_rng(seed)
    for it in range(ops):
        op = rng.integers(5)
        if op == 0:
            r = ins.record()
            assert max_rel_err(host(lay.step(to_dev(r))), ref.step(r), ref.scale) <= TOL, it
            pm.step()
        elif op in (1, 2):
            T = int(rng.integers(1, T_max + 1))
            d = ins.drafts(T)
            assert max_rel_err(host(lay.verify(to_dev(d))), ref.verify(d), ref.scale) <= TOL, it
            pm.verify(T)
            acc = rng.integers(0, T + 1, size=shape.batch).astype(np.int32)
            if op == 2 and it % 3 == 0:
                acc[-1] = -1                             # out of range: clamped to 0, status bit
            lay.commit(torch.from_numpy(acc).cuda())
            ref.commit(acc)
            pm.commit(acc)
        elif op == 4:
            # verify -> flush -> commit: the flush discards the pending drafts, so the
            # commit advances nothing (and flags the counts it clamps)
            T = int(rng.integers(1, T_max + 1))
            d = ins.drafts(T)
            assert max_rel_err(host(lay.verify(to_dev(d))), ref.verify(d), ref.scale) <= TOL, it
            pm.verify(T)
            mask = rng.integers(0, 2, size=shape.batch).astype(np.uint8)
            lay.flush(torch.from_numpy(mask).cuda())
            ref.flush(mask)
            pm.flush(mask.astype(bool))
            acc = rng.integers(0, T + 1, size=shape.batch).astype(np.int32)
            lay.commit(torch.from_numpy(acc).cuda())
            ref.commit(acc)
            pm.commit(acc)
        else:
            mask = rng.integers(0, 2, size=shape.batch).astype(np.uint8)
            lay.flush(torch.from_numpy(mask).cuda())
            pm.flush(mask.astype(bool))
        pos, ck = pointers_host(lay)
        assert np.array_equal(pos, pm.pos) and np.array_equal(ck, pm.ckpt_pos), it
        assert lay.status == pm.status, it
    lay.flush()
    assert ckpt_rel_err(host(lay.checkpoint), ref.state) <= TOL


@pytest.mark.parametrize("shape,T_max", [
    (LayerShape("gdn", 4, 3, 64, 32, 3, 6), 6),
    (LayerShape("gdn", 3, 4, 128, 128, 4, 16), 8),
    (LayerShape("gdn", 2, 3, 128, 128, 3, 16), 16),  # T = L: four passes of drafts, a fold before most verifies
    (LayerShape("gdn", 3, 2, 64, 128, 2, 12), 11),   # one row block per wave, three passes, L not a power of 2
    (LayerShape("gdn", 2, 3, 128, 32, 3, 8), 8),     # d_k = 32
])
def test_speculative_sequence(shape, T_max):
    _spec_run(shape, seed=13, ops=60, T_max=T_max)


def test_full_size_sampled():
    """Gated DeltaNet layer at batch 256 (32 heads, d_k = d_v = 128, L = 16), sampled sequences."""
    import torch
    shape = WORKLOADS["gdn_b256_h32_d128_l16"]
    announce("gdn full size", shape)
    ins = InputStream(shape, 2)
    lay = _layer(shape)
    sample = np.array([0, 129, 255])
    ref = StepwiseSession("gdn", np.zeros((len(sample), shape.heads, shape.head_dim, shape.state_dim)))
    worst = 0.0
    for t in range(2 * shape.window + 3):
        r = ins.record()
        y = lay.step(to_dev(r))
        worst = max(worst, max_rel_err(host(y[torch.from_numpy(sample).cuda()]), ref.step(take_batch(r, sample)), ref.scale))
    pos, ck = pointers_host(lay)
    assert np.all(pos == 2 * shape.window + 3) and np.all(ck == 2 * shape.window)
    assert worst <= TOL, worst
    lay.flush()
    assert ckpt_rel_err(host(lay.checkpoint[torch.from_numpy(sample).cuda()]), ref.state) <= TOL


def test_full_size_verify_sampled():
    import torch
    shape = WORKLOADS["gdn_b256_h32_d128_l16"]
    T = 8
    announce("gdn full-size verify", shape, "T", T)
    ins = InputStream(shape, 4)
    lay = _layer(shape, max_draft=T)
    pm = PointerMachine(shape.batch, shape.window)
    sample = np.array([3, 200])
    ref = StepwiseSession("gdn", np.zeros((len(sample), shape.heads, shape.head_dim, shape.state_dim)))
    worst = 0.0
    for it in range(5):
        d = ins.drafts(T)
        y = lay.verify(to_dev(d))
        pm.verify(T)
        worst = max(worst, max_rel_err(host(y[torch.from_numpy(sample).cuda()]), ref.verify(take_batch(d, sample)), ref.scale))
        acc = ins.accepted(T)
        lay.commit(torch.from_numpy(acc).cuda())
        pm.commit(acc)
        ref.commit(acc[sample])
        pos, ck = pointers_host(lay)
        assert np.array_equal(pos, pm.pos) and np.array_equal(ck, pm.ckpt_pos)
    assert worst <= TOL, worst


def test_conventional_and_snapshot_baselines():
    import torch
    from hybrid_model_ssm_replay_amd.layer import ConvLayer, SnapshotLayer
    shape = LayerShape("gdn", 3, 4, 128, 128, 4, 8)
    announce("gdn baselines", shape)
    ins = InputStream(shape, 8)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    conv = ConvLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, state0=S0)
    snap = SnapshotLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, 8, state0=S0)
    ref = StepwiseSession("gdn", S0)
    ref2 = StepwiseSession("gdn", S0)
    for _ in range(5):
        r = ins.record()
        assert max_rel_err(host(conv.step(to_dev(r))), ref.step(r), ref.scale) <= TOL
    assert ckpt_rel_err(host(conv.state), ref.state) <= TOL
    for T in (8, 2, 5):
        d = ins.drafts(T)
        assert max_rel_err(host(snap.verify(to_dev(d))), ref2.verify(d), ref2.scale) <= TOL
        acc = ins.accepted(T)
        snap.commit(torch.from_numpy(acc).cuda())
        ref2.commit(acc)
        assert ckpt_rel_err(host(snap.state()), ref2.state) <= TOL


def test_snapshot_baseline_large_lds():
    """T = 16 drafts at d_v = d_k = 128: the staged inputs take 72 KiB of LDS per
    workgroup, above the default dynamic limit, which the launch raises."""
    import torch
    from hybrid_model_ssm_replay_amd.layer import SnapshotLayer
    shape = LayerShape("gdn", 2, 3, 128, 128, 3, 16)
    announce("gdn snapshot T=16", shape)
    ins = InputStream(shape, 11)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    snap = SnapshotLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, 16, state0=S0)
    ref = StepwiseSession("gdn", S0)
    for T in (16, 9):
        d = ins.drafts(T)
        assert max_rel_err(host(snap.verify(to_dev(d))), ref.verify(d), ref.scale) <= TOL
        acc = ins.accepted(T)
        snap.commit(torch.from_numpy(acc).cuda())
        ref.commit(acc)
        assert ckpt_rel_err(host(snap.state()), ref.state) <= TOL


def test_decay_skip_matches_oracle():
    """REPLAY_FLAG_DECAY_SKIP on Gated DeltaNet heads: heads whose window
    log-decay falls below ln 2^-24 drop the checkpoint term (reading: see
    oracle/gdn.py).  Heads 0 and 2 get strong decays (alpha = e^-30: below the
    threshold from the first record; alpha ~ e^-2.5: from about the seventh),
    head 1 the usual ones.  Against ReplaySession with the same rule (and the
    exact form) through steps, folds, verifies, commits and a flush."""
    import torch
    from hybrid_model_ssm_replay_amd import binding as B
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    shape = LayerShape("gdn", 3, 4, 128, 128, 4, 8)
    announce("gdn decay skip", shape)
    ins = InputStream(shape, 19)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    lay = ReplayLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      max_draft=4, ckpt0=S0, flags=B.FLAG_DECAY_SKIP)
    skip = ReplaySession("gdn", S0, shape.window, decay_skip=True)
    exact = ReplaySession("gdn", S0, shape.window)

    def strong(r):
        r["alpha"][..., 0] = np.float32(np.exp(-30.0))
        r["alpha"][..., 2] = np.float32(np.exp(-2.5))
        return r

    rng = np.random.default_rng(19)
    worst_skip = worst_exact = 0.0
    for it in range(40):
        if it % 7 == 6:
            T = int(rng.integers(1, 5))
            d = strong(ins.drafts(T))
            y = host(lay.verify(to_dev(d)))
            ys, ye = skip.verify(d), exact.verify(d)
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            skip.commit(acc)
            exact.commit(acc)
        elif it == 20:
            lay.flush()
            skip.flush()
            exact.flush()
            continue
        else:
            r = strong(ins.record())
            y = host(lay.step(to_dev(r)))
            ys, ye = skip.step(r), exact.step(r)
        worst_skip = max(worst_skip, max_rel_err(y, ys, skip.scale))
        worst_exact = max(worst_exact, max_rel_err(y, ye, exact.scale))
    lay.flush()
    skip.flush()
    torch.cuda.synchronize()
    print(f"[gdn skip] vs skip rule {worst_skip:.2e}, vs exact {worst_exact:.2e}")
    assert worst_skip <= TOL, worst_skip
    assert worst_exact <= TOL, worst_exact
    assert ckpt_rel_err(host(lay.checkpoint), skip.ckpt) <= TOL
    assert lay.status == 0
