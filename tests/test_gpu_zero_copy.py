"""Zero-copy append (REPLAY_FLAG_RECORDS_IN_RING) on the GPU against the CPU oracle.

The test plays the producer: before each step or verify it asks the library
for the ring slot of each sequence's next record (replay_record_slots), writes
the fields the ring keeps (Mamba-2 x, B, dt; GDN k, alpha, beta) into those
slots through the views replay_ring_fields describes, and passes the call only
the other fields.  The results must equal those of the copying calls: outputs
and checkpoints within 1e-4 of the float64 stepwise definition, pointers and
status bit-exact (split-precision pairs: the bars of tests/test_gpu_split.py).
"""
import numpy as np
import pytest

from _gpu import announce, ckpt_rel_err, host, pointers_host, to_dev
from _metrics import max_rel_err
from oracle.pointers import PointerMachine
from oracle.session import FMT_F32, FMT_F4E2M1_B16, SplitReplaySession, StepwiseSession
from synth import InputStream, LayerShape

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _flags(bf16=False):
    from hybrid_model_ssm_replay_amd import binding as B
    return B.FLAG_RECORDS_IN_RING | (B.FLAG_BF16_RECORDS if bf16 else 0)


def _layer(shape, ins, max_draft, ckpt0, bf16=False, **kw):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    extra = {"groups": shape.groups, "A": ins.params["A"], "D": ins.params["D"]} if shape.kind == "mamba2" else {}
    return ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       max_draft=max_draft, ckpt0=ckpt0, flags=_flags(bf16), **extra, **kw)


def _produce(lay, rec):
    """Write the ring-kept fields of a device record ([batch, ...]) or of drafts
    ([batch, T, ...]) into ring slots (slot + i) mod slots, as a producer would."""
    import torch
    f = lay.ring_fields()
    slots = lay.record_slots().long()
    bi = torch.arange(slots.numel(), device=slots.device)
    first = "x" if "x" in f else "k"
    n = f[first].shape[0]
    drafts = rec[first].dim() == 4
    T = rec[first].shape[1] if drafts else 1
    for i in range(T):
        sl = (slots + i) % n
        pick = (lambda t: t[:, i]) if drafts else (lambda t: t)  # noqa: E731
        f[first][sl, bi] = pick(rec[first])
        if "B" in f:
            f["B"][bi, :, sl] = pick(rec["B"])
            f["dt"][bi, :, sl] = pick(rec["dt"])
        else:
            f["alpha"][bi, :, sl] = pick(rec["alpha"])
            f["beta"][bi, :, sl] = pick(rec["beta"])


def _spec_run(shape, seed, ops, T_max, bf16=False):
    import torch
    announce("zero-copy speculative", shape, "seed", seed, "bf16", bf16)
    ins = InputStream(shape, seed, bf16_vectors=bf16)
    S0 = ins.initial_state(zeros=False, scale=0.5 if shape.kind == "mamba2" else 0.3)
    lay = _layer(shape, ins, T_max, S0, bf16)
    ref = StepwiseSession(shape.kind, S0, ins.params)
    pm = PointerMachine(shape.batch, shape.window)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for it in range(ops):
        op = rng.integers(4)
        if op == 0:
            r = ins.record()
            dr = to_dev(r, bf16)
            _produce(lay, dr)
            worst = max(worst, max_rel_err(host(lay.step(dr)), ref.step(r), ref.scale))
            pm.step()
        elif op in (1, 2):
            T = int(rng.integers(1, T_max + 1))
            d = ins.drafts(T)
            dd = to_dev(d, bf16)
            _produce(lay, dd)
            worst = max(worst, max_rel_err(host(lay.verify(dd)), ref.verify(d), ref.scale))
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
    (LayerShape("mamba2", 3, 8, 64, 128, 2, 16), 8),    # headline head shape
    (LayerShape("mamba2", 2, 4, 64, 128, 2, 16), 16),   # T = L: the drafts fill the other L slots
    (LayerShape("mamba2", 5, 3, 32, 16, 1, 7), 7),      # ragged, odd window
    (LayerShape("mamba2", 2, 6, 128, 32, 3, 5), 5),     # P = 128
])
def test_mamba2(shape, T_max):
    _spec_run(shape, seed=41, ops=50, T_max=T_max)


@pytest.mark.parametrize("shape,T_max", [
    (LayerShape("gdn", 3, 4, 128, 128, 4, 8), 8),
    (LayerShape("gdn", 2, 3, 64, 32, 3, 16), 16),       # d_k = 32, T = L
    (LayerShape("gdn", 3, 5, 128, 64, 5, 11), 11),      # odd window
])
def test_gdn(shape, T_max):
    _spec_run(shape, seed=42, ops=50, T_max=T_max)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_with_bf16_records(kind):
    shape = LayerShape(kind, 3, 8, 64, 128, 2, 16) if kind == "mamba2" else LayerShape(kind, 3, 4, 128, 128, 4, 8)
    _spec_run(shape, seed=43, ops=40, T_max=8, bf16=True)


def test_gdn_split_precision():
    """f32 checkpoint + e2m1 read copy with the records in the ring: the
    re-solving fold reads the producer's keys and scalars and its own v."""
    import torch
    shape = LayerShape("gdn", 2, 3, 128, 128, 3, 4)
    announce("zero-copy split", shape)
    ins = InputStream(shape, 44)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    lay = _layer(shape, ins, 3, S0, ckpt_fmt=FMT_F32, read_fmt=FMT_F4E2M1_B16, seed=77)
    sess = SplitReplaySession("gdn", S0, shape.window, None, FMT_F32, FMT_F4E2M1_B16, seed=77)
    rng = np.random.default_rng(44)
    worst_pre = worst_post = 0.0
    for t in range(17):
        if t in (6, 11):
            T = int(rng.integers(1, 4))
            d = ins.drafts(T)
            dd = to_dev(d)
            _produce(lay, dd)
            e = max_rel_err(host(lay.verify(dd)), sess.verify(d), sess.scale)
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            sess.commit(acc)
        else:
            r = ins.record()
            dr = to_dev(r)
            _produce(lay, dr)
            e = max_rel_err(host(lay.step(dr)), sess.step(r), sess.scale)
        if t < shape.window:
            worst_pre = max(worst_pre, e)
        else:
            worst_post = max(worst_post, e)
    assert worst_pre <= TOL, worst_pre
    assert worst_post <= 2e-2, worst_post


def test_mamba2_with_decay_skip():
    """Zero-copy steps and verifies with REPLAY_FLAG_DECAY_SKIP, against the oracle
    session with the same rule."""
    import torch
    from hybrid_model_ssm_replay_amd import binding as B
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from oracle.session import ReplaySession
    shape = LayerShape("mamba2", 3, 8, 64, 128, 2, 16)
    announce("zero-copy decay skip", shape)
    ins = InputStream(shape, 45)
    params = {"A": ins.params["A"].copy(), "D": ins.params["D"]}
    params["A"][:3] = np.array([-80.0, -40.0, -25.0], np.float32)  # heads that skip within a window
    S0 = ins.initial_state(zeros=False, scale=0.5)
    lay = ReplayLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      groups=shape.groups, max_draft=6, A=params["A"], D=params["D"], ckpt0=S0,
                      flags=B.FLAG_DECAY_SKIP | B.FLAG_RECORDS_IN_RING)
    skip = ReplaySession("mamba2", S0, shape.window, params, decay_skip=True)
    rng = np.random.default_rng(45)
    worst = 0.0
    for it in range(45):
        if it % 7 == 6:
            T = int(rng.integers(1, 7))
            d = ins.drafts(T)
            dd = to_dev(d)
            _produce(lay, dd)
            worst = max(worst, max_rel_err(host(lay.verify(dd)), skip.verify(d), skip.scale))
            acc = ins.accepted(T)
            lay.commit(torch.from_numpy(acc).cuda())
            skip.commit(acc)
        else:
            r = ins.record()
            dr = to_dev(r)
            _produce(lay, dr)
            worst = max(worst, max_rel_err(host(lay.step(dr)), skip.step(r), skip.scale))
    lay.flush()
    skip.flush()
    assert worst <= TOL, worst
    assert ckpt_rel_err(host(lay.checkpoint), skip.ckpt) <= TOL
    assert lay.status == 0
