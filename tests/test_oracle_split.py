"""Pins for the split-precision replay oracle.

The pages state what separating the two precisions does: the read copy's
rounding never re-enters the recurrence, so its error does not grow with
generation length, while a shared low-precision checkpoint feeds its rounding
back and accumulates error; an FP16 recurrence with stochastic rounding tracks
FP32 closely [P1, Interpretation 4; P1, Perspective 2; P3, Interpretation 3;
P3, Perspective 2].  These tests check exactly those statements on a small
Gated DeltaNet layer whose heads decay slowly (long memory), against the
float64 stepwise definition.
"""
import numpy as np
import pytest

from oracle.session import (FMT_F16_SR, FMT_F32, FMT_F4E2M1_B16, FMT_F8E4M3, ReplaySession, SplitReplaySession,
                            StepwiseSession, decode_state, encode_state)
from synth import InputStream, LayerShape

SHAPE = LayerShape("gdn", 1, 2, 32, 32, 2, 16)


def _errors(cf, rf, steps, decay_scale=0.01, seed=4):
    ins = InputStream(SHAPE, seed)
    S0 = ins.initial_state(zeros=True)
    sp = SplitReplaySession("gdn", S0, SHAPE.window, None, cf, rf, seed=11)
    ref = StepwiseSession("gdn", S0)
    errs = []
    for _ in range(steps):
        r = ins.record()
        r["alpha"] = np.exp(np.log(r["alpha"]) * decay_scale).astype(np.float32)
        y, yr = sp.step(r), ref.step(r)
        errs.append(np.max(np.abs(y - yr)) / np.max(np.abs(yr)))
    return np.array(errs)


@pytest.mark.slow
def test_shared_low_precision_accumulates_split_does_not():
    split = _errors(FMT_F32, FMT_F4E2M1_B16, 1536)
    shared = _errors(FMT_F4E2M1_B16, FMT_F4E2M1_B16, 1536)
    early, late = slice(16, 64), slice(768, 1536)
    assert late.stop <= len(split)
    growth_split = split[late].mean() / split[early].mean()
    growth_shared = shared[late].mean() / shared[early].mean()
    assert growth_split < 1.25, growth_split
    assert growth_shared > 1.4, growth_shared
    assert shared[late].mean() > 1.5 * split[late].mean()


@pytest.mark.slow
def test_fp16_sr_recurrence_tracks_fp32():
    fp16 = _errors(FMT_F16_SR, FMT_F16_SR, 768)
    fp8 = _errors(FMT_F8E4M3, FMT_F8E4M3, 768)
    assert fp16[256:].mean() < 1e-3
    assert fp16[256:].mean() < 0.05 * fp8[256:].mean()


def test_f32_storage_is_the_replay_form():
    ins = InputStream(LayerShape("gdn", 2, 2, 32, 32, 2, 4), 1)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    sp = SplitReplaySession("gdn", S0, 4, None, FMT_F32, FMT_F32)
    rp = ReplaySession("gdn", S0, 4)
    for _ in range(13):
        r = ins.record()
        np.testing.assert_allclose(sp.step(r), rp.step(r), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("fmt", [FMT_F32, FMT_F16_SR, FMT_F8E4M3, FMT_F4E2M1_B16])
def test_encode_decode_error_bounds(fmt):
    rng = np.random.default_rng(5)
    S = rng.standard_normal((2, 32, 32)).astype(np.float32)
    D = decode_state(encode_state(S, fmt, seed=3, b=1, ckpt_pos=9), fmt)
    rel = np.abs(D - S) / np.maximum(np.abs(S), 1e-30)
    bound = {FMT_F32: 0.0, FMT_F16_SR: 2.0 ** -10, FMT_F8E4M3: 2.0 ** -4}.get(fmt)
    if bound is not None:
        big = np.abs(S) > 2.0 ** -5                      # away from the subnormal ranges
        assert np.all(rel[big] <= bound + 1e-12)
    else:
        # e2m1: at most one grid step (2 s) per element of a block with scale s ~ amax / 6
        blk = S.reshape(2, 32, 2, 16)
        amax = np.abs(blk).max(-1, keepdims=True)
        err = np.abs(D - S).reshape(2, 32, 2, 16)
        assert np.all(err <= amax / 6 * 1.07 * 2 + 1e-12)


def _kind_inputs(kind, seed):
    shape = LayerShape(kind, 2, 2, 16, 32, 1 if kind == "mamba2" else 2, 4)
    ins = InputStream(shape, seed)
    return shape, ins, ins.initial_state(zeros=False, scale=0.3)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("cf,rf", [(FMT_F32, FMT_F4E2M1_B16), (FMT_F16_SR, FMT_F4E2M1_B16),
                                   (FMT_F4E2M1_B16, FMT_F4E2M1_B16)])
def test_fold_step_outputs_come_from_the_exact_fold(kind, cf, rf):
    """The step that folds outputs from the fold result, not from the read copy
    [P3, Perspective, paragraph 2]: at the first fold both sessions fold the same
    decoded checkpoint with the same records, so in float64 that output equals
    the exact replay form's to rounding, while the outputs of the steps around it
    read the approximate copy and do not."""
    shape, ins, S0 = _kind_inputs(kind, 3)
    sp = SplitReplaySession(kind, S0, shape.window, ins.params, cf, rf, seed=5)
    start = np.stack([sp.recurrence_state(b) for b in range(shape.batch)])
    rp = ReplaySession(kind, start, shape.window, ins.params)
    errs = []
    for _ in range(shape.window + 3):
        r = ins.record()
        y, ye = sp.step(r), rp.step(r)
        errs.append(np.max(np.abs(y - ye)) / np.max(np.abs(ye)))
    fold_step = shape.window                              # the (L+1)-th step folds first
    assert errs[fold_step] <= 1e-12, errs
    # the steps after it read the encoded fold result (and, with a separate read
    # copy, so do the steps before it: a shared copy starts as the checkpoint)
    approx = errs[fold_step + 1:] + (errs[:fold_step] if rf != cf else [])
    assert min(approx) > 1e-4, errs


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_verify_fold_first_outputs_come_from_the_exact_fold(kind):
    shape, ins, S0 = _kind_inputs(kind, 8)
    sp = SplitReplaySession(kind, S0, shape.window, ins.params, FMT_F32, FMT_F4E2M1_B16, seed=5)
    rp = ReplaySession(kind, S0, shape.window, ins.params)
    for _ in range(3):
        r = ins.record()
        sp.step(r), rp.step(r)
    d = ins.drafts(3)                                     # 3 + 3 > 4: folds first
    y, ye = sp.verify(d), rp.verify(d)
    assert np.max(np.abs(y - ye)) / np.max(np.abs(ye)) <= 1e-12
    sp.commit(np.array([1, 3])), rp.commit(np.array([1, 3]))
    r = ins.record()                                      # a non-fold step reads the e2m1 copy again
    y, ye = sp.step(r), rp.step(r)
    assert np.max(np.abs(y - ye)) / np.max(np.abs(ye)) > 1e-4
