"""Mamba-2 replay decode on the GPU against the CPU oracle.

Outputs: max relative error <= 1e-4 per output vector (one head of one
sequence at one token; tests/_metrics.py) against the float64 stepwise
definition.  Pointers (pos, ckpt_pos), fold positions and status bits:
bit-exact against the oracle's pointer machine.  Checkpoints after a fold:
<= 1e-4 relative to the oracle's exact state.
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


def _layer(shape, ins, max_draft=0, ckpt0=None):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    return ReplayLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       groups=shape.groups, max_draft=max_draft, A=ins.params["A"], D=ins.params["D"],
                       ckpt0=ckpt0)


def _run_steps(shape, seed, steps, ckpt0_zero=True):
    announce("mamba2 steps", shape, "seed", seed, "steps", steps)
    import torch
    ins = InputStream(shape, seed)
    S0 = ins.initial_state(zeros=ckpt0_zero, scale=0.5)
    lay = _layer(shape, ins, ckpt0=S0)
    ref = StepwiseSession("mamba2", S0, ins.params)
    rep = ReplaySession("mamba2", S0, shape.window, ins.params)
    worst = 0.0
    for t in range(steps):
        r = ins.record()
        y = host(lay.step(to_dev(r)))
        y_ref = ref.step(r)
        rep.step(r)
        worst = max(worst, max_rel_err(y, y_ref, ref.scale))
        pos, ck = pointers_host(lay)
        assert np.array_equal(pos, rep.ptr.pos) and np.array_equal(ck, rep.ptr.ckpt_pos), t
    torch.cuda.synchronize()
    assert worst <= TOL, worst
    # the checkpoint equals the oracle's fold (exact state at ckpt_pos)
    assert ckpt_rel_err(host(lay.checkpoint), rep.ckpt) <= TOL
    assert lay.status == 0
    return worst


def test_tiny_every_step():
    _run_steps(WORKLOADS["mamba2_b2_h4_p16_n16_l4"], seed=0, steps=64)


@pytest.mark.parametrize("shape", [
    LayerShape("mamba2", 3, 8, 64, 128, 2, 5),     # several tiles, odd window, ragged step count
    LayerShape("mamba2", 2, 6, 128, 32, 3, 16),    # two row blocks per wave
    LayerShape("mamba2", 1, 4, 48, 64, 4, 1),      # L = 1: conventional decoding, fold every step
    LayerShape("mamba2", 5, 3, 32, 16, 1, 7),      # batch*heads not a multiple of 8
])
def test_shapes_ragged(shape):
    _run_steps(shape, seed=11, steps=2 * shape.window + 3, ckpt0_zero=False)


def _spec_run(shape, seed, ops, T_max):
    import torch
    announce("mamba2 speculative", shape, "seed", seed)
    ins = InputStream(shape, seed)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    lay = _layer(shape, ins, max_draft=T_max, ckpt0=S0)
    ref = StepwiseSession("mamba2", S0, ins.params)
    pm = PointerMachine(shape.batch, shape.window)
    rng = np.random.default_rng(seed)
    for it in range(ops):
        op = rng.integers(5)
        if op == 0:
            r = ins.record()
            y = host(lay.step(to_dev(r)))
            assert max_rel_err(y, ref.step(r), ref.scale) <= TOL, it
            pm.step()
        elif op in (1, 2):
            T = int(rng.integers(1, T_max + 1))
            d = ins.drafts(T)
            y = host(lay.verify(to_dev(d)))
            assert max_rel_err(y, ref.verify(d), ref.scale) <= TOL, it
            pm.verify(T)
            acc = rng.integers(0, T + 1, size=shape.batch).astype(np.int32)
            if op == 2 and it % 3 == 0:
                acc[0] = T + 2                          # out of range: clamped, status bit
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
    pm.flush()
    assert ckpt_rel_err(host(lay.checkpoint), ref.state) <= TOL


@pytest.mark.parametrize("shape,T_max", [
    (LayerShape("mamba2", 4, 4, 32, 64, 2, 6), 6),
    (LayerShape("mamba2", 3, 8, 64, 128, 8, 16), 8),
    (LayerShape("mamba2", 2, 2, 16, 16, 1, 3), 3),
    (LayerShape("mamba2", 2, 2, 16, 32, 1, 12), 12),  # one wave per head, more drafts than 64 / 16
    (LayerShape("mamba2", 2, 4, 64, 128, 2, 16), 16),  # T = L: four passes of drafts
])
def test_speculative_sequence(shape, T_max):
    _spec_run(shape, seed=5, ops=60, T_max=T_max)


def test_verify_writes_no_state_without_fold():
    import torch
    shape = LayerShape("mamba2", 2, 4, 32, 32, 2, 8)
    announce("mamba2 verify no-write", shape)
    ins = InputStream(shape, 3)
    lay = _layer(shape, ins, max_draft=4, ckpt0=ins.initial_state(zeros=False))
    for _ in range(3):
        lay.step(to_dev(ins.record()))
    before = lay.checkpoint.clone()
    lay.verify(to_dev(ins.drafts(4)))
    lay.commit(torch.zeros(shape.batch, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(before, lay.checkpoint)


def test_deterministic_bytes():
    import torch
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 4)
    announce("mamba2 determinism", shape)
    outs = []
    for _ in range(2):
        ins = InputStream(shape, 21)
        lay = _layer(shape, ins, ckpt0=ins.initial_state(zeros=False))
        ys = [lay.step(to_dev(ins.record())) for _ in range(9)]
        torch.cuda.synchronize()
        outs.append((torch.stack(ys).cpu(), lay.checkpoint.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_bad_pointers_are_flagged_and_skipped():
    import torch
    shape = LayerShape("mamba2", 2, 4, 16, 16, 1, 4)
    announce("mamba2 bad pointers", shape)
    ins = InputStream(shape, 4)
    lay = _layer(shape, ins)
    lay.step(to_dev(ins.record()))
    pos, ck = lay.pointers()
    pos[1] = 100                                       # count = 100 > L for sequence 1
    y = torch.full((shape.batch, shape.heads, shape.head_dim), 7.0, device="cuda")
    lay.step(to_dev(ins.record()), y=y)
    pos2, ck2 = pointers_host(lay)
    assert lay.status & 0x2
    assert pos2[1] == 100 and ck2[1] == 0 and pos2[0] == 2
    assert torch.all(y[1] == 7.0)                       # skipped sequence: output untouched


def test_full_size_sampled():
    """The 4 MiB-per-sequence layer at batch 256, checked on sampled sequences."""
    import torch
    shape = WORKLOADS["mamba2_b256_h128_p64_n128_g8_l16"]
    announce("mamba2 full size", shape)
    ins = InputStream(shape, 1)
    lay = _layer(shape, ins)
    sample = np.array([0, 77, 200, 255])
    ref = StepwiseSession("mamba2", np.zeros((len(sample), shape.heads, shape.head_dim, shape.state_dim)), ins.params)
    worst = 0.0
    for t in range(2 * shape.window + 3):
        r = ins.record()
        y = lay.step(to_dev(r))
        y_s = host(y[torch.from_numpy(sample).cuda()])
        worst = max(worst, max_rel_err(y_s, ref.step(take_batch(r, sample)), ref.scale))
    pos, ck = pointers_host(lay)
    assert np.all(pos == 2 * shape.window + 3) and np.all(ck == 2 * shape.window)
    assert worst <= TOL, worst
    lay.flush()
    ck_s = host(lay.checkpoint[torch.from_numpy(sample).cuda()])
    assert ckpt_rel_err(ck_s, ref.state) <= TOL


@pytest.mark.parametrize("T", [4, 8])
def test_full_size_verify_sampled(T):
    """Speculative verify on the batch-512 layer; sampled sequences, pointers in full."""
    import torch
    shape = WORKLOADS["mamba2_b512_h128_p64_n128_g8_l16"]
    announce("mamba2 full-size verify", shape, "T", T)
    ins = InputStream(shape, 3)
    lay = _layer(shape, ins, max_draft=T)
    pm = PointerMachine(shape.batch, shape.window)
    sample = np.array([1, 300, 511])
    ref = StepwiseSession("mamba2", np.zeros((len(sample), shape.heads, shape.head_dim, shape.state_dim)), ins.params)
    worst = 0.0
    for it in range(6):
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


def test_conventional_baseline():
    from hybrid_model_ssm_replay_amd.layer import ConvLayer
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 1)
    announce("mamba2 conventional", shape)
    ins = InputStream(shape, 8)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    conv = ConvLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, groups=shape.groups,
                     A=ins.params["A"], D=ins.params["D"], state0=S0)
    ref = StepwiseSession("mamba2", S0, ins.params)
    for _ in range(7):
        r = ins.record()
        assert max_rel_err(host(conv.step(to_dev(r))), ref.step(r), ref.scale) <= TOL
    assert ckpt_rel_err(host(conv.state), ref.state) <= TOL


def test_snapshot_baseline():
    import torch
    from hybrid_model_ssm_replay_amd.layer import SnapshotLayer
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 8)
    announce("mamba2 snapshot", shape)
    ins = InputStream(shape, 9)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    snap = SnapshotLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, 8, groups=shape.groups,
                         A=ins.params["A"], D=ins.params["D"], state0=S0)
    ref = StepwiseSession("mamba2", S0, ins.params)
    for T in (8, 3, 5, 8):
        d = ins.drafts(T)
        assert max_rel_err(host(snap.verify(to_dev(d))), ref.verify(d), ref.scale) <= TOL
        acc = ins.accepted(T)
        snap.commit(torch.from_numpy(acc).cuda())
        ref.commit(acc)
        assert ckpt_rel_err(host(snap.state()), ref.state) <= TOL


def test_snapshot_baseline_large_lds():
    """T = 16 drafts at P = 128 (four waves): the staged inputs take 72 KiB of LDS
    per workgroup, above the default dynamic limit, which the launch raises."""
    import torch
    from hybrid_model_ssm_replay_amd.layer import SnapshotLayer
    shape = LayerShape("mamba2", 2, 4, 128, 128, 2, 16)
    announce("mamba2 snapshot T=16", shape)
    ins = InputStream(shape, 10)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    snap = SnapshotLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, 16, groups=shape.groups,
                         A=ins.params["A"], D=ins.params["D"], state0=S0)
    ref = StepwiseSession("mamba2", S0, ins.params)
    for T in (16, 7):
        d = ins.drafts(T)
        assert max_rel_err(host(snap.verify(to_dev(d))), ref.verify(d), ref.scale) <= TOL
        acc = ins.accepted(T)
        snap.commit(torch.from_numpy(acc).cuda())
        ref.commit(acc)
        assert ckpt_rel_err(host(snap.state()), ref.state) <= TOL


def test_decay_skip_matches_oracle():
    """REPLAY_FLAG_DECAY_SKIP: steps, verifies, commits and a flush against the
    oracle session with the same rule (heads whose window decay is below 2^-24
    drop the checkpoint term), and against the exact method (the dropped terms
    are below float32 rounding)."""
    import torch
    from hybrid_model_ssm_replay_amd import binding as B
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 16)
    announce("mamba2 decay skip", shape)
    ins = InputStream(shape, 9)
    params = {"A": ins.params["A"].copy(), "D": ins.params["D"]}
    params["A"][:3] = np.array([-80.0, -40.0, -25.0], np.float32)  # heads that skip within a window
    S0 = ins.initial_state(zeros=False, scale=0.5)
    lay = ReplayLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      groups=shape.groups, max_draft=6, A=params["A"], D=params["D"], ckpt0=S0,
                      flags=B.FLAG_DECAY_SKIP)
    skip = ReplaySession("mamba2", S0, shape.window, params, decay_skip=True)
    exact = ReplaySession("mamba2", S0, shape.window, params)
    rng = np.random.default_rng(9)
    worst_skip = worst_exact = 0.0
    skipped_any = False
    for it in range(50):
        if it % 7 == 6:
            T = int(rng.integers(1, 7))
            d = ins.drafts(T)
            y = host(lay.verify(to_dev(d)))
            ys, ye = skip.verify(d), exact.verify(d)
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            skip.commit(acc)
            exact.commit(acc)
        else:
            r = ins.record()
            y = host(lay.step(to_dev(r)))
            ys, ye = skip.step(r), exact.step(r)
        worst_skip = max(worst_skip, max_rel_err(y, ys, skip.scale))
        worst_exact = max(worst_exact, max_rel_err(y, ye, exact.scale))
        skipped_any = skipped_any or not np.allclose(ys, ye, rtol=0, atol=0)
    lay.flush()
    skip.flush()
    torch.cuda.synchronize()
    assert skipped_any  # the rule did drop terms in this run
    assert worst_skip <= TOL, worst_skip
    assert worst_exact <= TOL, worst_exact
    assert ckpt_rel_err(host(lay.checkpoint), skip.ckpt) <= TOL
    assert lay.status == 0
