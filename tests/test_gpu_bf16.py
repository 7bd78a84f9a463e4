"""bf16 records (REPLAY_FLAG_BF16_RECORDS) on the GPU against the CPU oracle.

The record vector fields (Mamba-2 x, B, C; GDN q, k, v) are drawn and then
rounded to bf16 values by the input generator; the GPU receives them as bf16
tensors (its ring keeps bf16 copies) and the oracle the same values in float64.
Widening bf16 to float32 is exact, so the method's results must meet the same
bars as with float32 records: outputs and checkpoints within 1e-4 of the
float64 stepwise definition, pointers and status bit-exact.  The split-precision
case uses the bars of tests/test_gpu_split.py.
"""
import numpy as np
import pytest

from _gpu import announce, ckpt_rel_err, host, pointers_host, to_dev
from _metrics import max_rel_err
from oracle.pointers import PointerMachine
from oracle.session import (FMT_F32, FMT_F4E2M1_B16, FMT_F4E2M1_CS, FMT_F8E4M3, SplitReplaySession,
                            StepwiseSession)
from synth import WORKLOADS, InputStream, LayerShape, take_batch

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _flag():
    from hybrid_model_ssm_replay_amd.binding import FLAG_BF16_RECORDS
    return FLAG_BF16_RECORDS


def _replay_layer(shape, ins, max_draft, ckpt0, **kw):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    extra = {"groups": shape.groups, "A": ins.params["A"], "D": ins.params["D"]} if shape.kind == "mamba2" else {}
    return ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       max_draft=max_draft, ckpt0=ckpt0, flags=_flag(), **extra, **kw)


def _spec_run(shape, seed, ops, T_max):
    """Random steps, verifies with commits (one clamped) and masked flushes."""
    import torch
    announce("bf16 speculative", shape, "seed", seed)
    ins = InputStream(shape, seed, bf16_vectors=True)
    S0 = ins.initial_state(zeros=False, scale=0.5 if shape.kind == "mamba2" else 0.3)
    lay = _replay_layer(shape, ins, T_max, S0)
    ref = StepwiseSession(shape.kind, S0, ins.params)
    pm = PointerMachine(shape.batch, shape.window)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for it in range(ops):
        op = rng.integers(4)
        if op == 0:
            r = ins.record()
            worst = max(worst, max_rel_err(host(lay.step(to_dev(r, bf16=True))), ref.step(r), ref.scale))
            pm.step()
        elif op in (1, 2):
            T = int(rng.integers(1, T_max + 1))
            d = ins.drafts(T)
            worst = max(worst, max_rel_err(host(lay.verify(to_dev(d, bf16=True))), ref.verify(d), ref.scale))
            pm.verify(T)
            acc = rng.integers(0, T + 1, size=shape.batch).astype(np.int32)
            if op == 2 and it % 3 == 0:
                acc[0] = T + 2                          # out of range: clamped, status bit
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
    assert worst <= TOL, worst
    lay.flush()
    pm.flush()
    assert ckpt_rel_err(host(lay.checkpoint), ref.state) <= TOL


@pytest.mark.parametrize("shape,T_max", [
    (LayerShape("mamba2", 3, 8, 64, 128, 2, 16), 8),    # headline head shape, two row blocks per wave
    (LayerShape("mamba2", 2, 4, 64, 128, 2, 16), 16),   # T = L: four passes of drafts
    (LayerShape("mamba2", 5, 3, 32, 16, 1, 7), 7),      # ragged: batch * heads not a multiple of 8
    (LayerShape("mamba2", 2, 6, 128, 32, 3, 5), 5),     # P = 128
])
def test_mamba2_speculative(shape, T_max):
    _spec_run(shape, seed=31, ops=50, T_max=T_max)


@pytest.mark.parametrize("shape,T_max", [
    (LayerShape("gdn", 3, 4, 128, 128, 4, 8), 8),
    (LayerShape("gdn", 2, 3, 64, 32, 3, 16), 16),       # d_k = 32, T = L
    (LayerShape("gdn", 3, 5, 128, 64, 5, 11), 11),      # odd window, d_k = 64
])
def test_gdn_speculative(shape, T_max):
    _spec_run(shape, seed=32, ops=50, T_max=T_max)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_baselines(kind):
    """Conventional step and snapshot verify with bf16 records."""
    import torch
    from hybrid_model_ssm_replay_amd.layer import ConvLayer, SnapshotLayer
    shape = LayerShape(kind, 3, 8, 64, 128, 2, 8) if kind == "mamba2" else LayerShape(kind, 3, 4, 128, 128, 4, 8)
    announce("bf16 baselines", shape)
    ins = InputStream(shape, 33, bf16_vectors=True)
    S0 = ins.initial_state(zeros=False, scale=0.4)
    extra = {"groups": shape.groups, "A": ins.params["A"], "D": ins.params["D"]} if kind == "mamba2" else {}
    conv = ConvLayer(kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, state0=S0, flags=_flag(),
                     **extra)
    snap = SnapshotLayer(kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, 8, state0=S0,
                         flags=_flag(), **extra)
    ref, ref2 = StepwiseSession(kind, S0, ins.params), StepwiseSession(kind, S0, ins.params)
    for _ in range(5):
        r = ins.record()
        assert max_rel_err(host(conv.step(to_dev(r, bf16=True))), ref.step(r), ref.scale) <= TOL
    assert ckpt_rel_err(host(conv.state), ref.state) <= TOL
    for T in (8, 3, 5):
        d = ins.drafts(T)
        assert max_rel_err(host(snap.verify(to_dev(d, bf16=True))), ref2.verify(d), ref2.scale) <= TOL
        acc = ins.accepted(T)
        snap.commit(torch.from_numpy(acc).cuda())
        ref2.commit(acc)
        assert ckpt_rel_err(host(snap.state()), ref2.state) <= TOL


@pytest.mark.parametrize("cf,rf", [(FMT_F32, FMT_F4E2M1_B16), (FMT_F8E4M3, FMT_F4E2M1_B16), (FMT_F32, FMT_F4E2M1_CS),
                                   (FMT_F4E2M1_B16, FMT_F4E2M1_B16)])
def test_gdn_split_precision(cf, rf):
    """Split-precision GDN with bf16 records (the buffered v is bf16 too):
    outputs within 1e-4 before the first fold and within one e2m1 step
    (2e-2, as for float32 records) after it."""
    import torch
    shape = LayerShape("gdn", 2, 3, 128, 128, 3, 4)
    announce("bf16 split", shape, cf, rf)
    ins = InputStream(shape, 34, bf16_vectors=True)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    lay = _replay_layer(shape, ins, 3, S0, ckpt_fmt=cf, read_fmt=rf, seed=77)
    sess = SplitReplaySession("gdn", S0, shape.window, None, cf, rf, seed=77)
    rng = np.random.default_rng(34)
    worst_pre = worst_post = 0.0
    for t in range(17):
        if t in (6, 11):
            T = int(rng.integers(1, 4))
            d = ins.drafts(T)
            e = max_rel_err(host(lay.verify(to_dev(d, bf16=True))), sess.verify(d), sess.scale)
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            sess.commit(acc)
        else:
            r = ins.record()
            e = max_rel_err(host(lay.step(to_dev(r, bf16=True))), sess.step(r), sess.scale)
        if t < shape.window:
            worst_pre = max(worst_pre, e)
        else:
            worst_post = max(worst_post, e)
    print(f"[bf16 split] cf={cf} rf={rf} pre-fold {worst_pre:.2e} post-fold {worst_post:.2e}")
    assert worst_pre <= TOL, worst_pre
    assert worst_post <= 2e-2, worst_post


def test_mamba2_full_size_sampled():
    """The bf16-record bench configuration (Mamba-2, 128 heads, P = 64, N = 128,
    8 groups, L = 16, batch 256): 20 steps (one fold) and a T = 8 verify, on 4
    sampled sequences."""
    import torch
    shape = WORKLOADS["mamba2_b256_h128_p64_n128_g8_l16"]
    announce("bf16 mamba2 full size", shape)
    ins = InputStream(shape, 35, bf16_vectors=True)
    lay = _replay_layer(shape, ins, 8, None)
    sample = np.array([0, 77, 128, 255])
    ref = StepwiseSession("mamba2", np.zeros((len(sample), shape.heads, shape.head_dim, shape.state_dim)),
                          ins.params)
    idx = torch.from_numpy(sample).cuda()
    worst = 0.0
    for _ in range(20):
        r = ins.record()
        y = lay.step(to_dev(r, bf16=True))
        worst = max(worst, max_rel_err(host(y[idx]), ref.step(take_batch(r, sample)), ref.scale))
    d = ins.drafts(8)
    y = lay.verify(to_dev(d, bf16=True))
    worst = max(worst, max_rel_err(host(y[idx]), ref.verify(take_batch(d, sample)), ref.scale))
    assert worst <= TOL, worst


def test_mamba2_with_decay_skip():
    """bf16 records with REPLAY_FLAG_DECAY_SKIP, against the oracle session with
    the same rule on the same bf16-valued inputs."""
    import torch
    from hybrid_model_ssm_replay_amd import binding as B
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from oracle.session import ReplaySession
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 16)
    announce("bf16 decay skip", shape)
    ins = InputStream(shape, 36, bf16_vectors=True)
    params = {"A": ins.params["A"].copy(), "D": ins.params["D"]}
    params["A"][:3] = np.array([-80.0, -40.0, -25.0], np.float32)  # heads that skip within a window
    S0 = ins.initial_state(zeros=False, scale=0.5)
    lay = ReplayLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      groups=shape.groups, max_draft=6, A=params["A"], D=params["D"], ckpt0=S0,
                      flags=B.FLAG_DECAY_SKIP | B.FLAG_BF16_RECORDS)
    skip = ReplaySession("mamba2", S0, shape.window, params, decay_skip=True)
    rng = np.random.default_rng(36)
    worst = 0.0
    for it in range(45):
        if it % 7 == 6:
            T = int(rng.integers(1, 7))
            d = ins.drafts(T)
            worst = max(worst, max_rel_err(host(lay.verify(to_dev(d, bf16=True))), skip.verify(d), skip.scale))
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            skip.commit(acc)
        else:
            r = ins.record()
            worst = max(worst, max_rel_err(host(lay.step(to_dev(r, bf16=True))), skip.step(r), skip.scale))
    lay.flush()
    skip.flush()
    assert worst <= TOL, worst
    assert ckpt_rel_err(host(lay.checkpoint), skip.ckpt) <= TOL
