"""Degenerate inputs on the GPU against the CPU oracle (the same 1e-4 bar).

* Decays far below float32's range: Mamba-2 heads with A = -16 and dt near 8
  (a window's log-decay near -2000) and GDN heads with alpha = 1e-30 (log-decay
  -69 per record).  Decays are formed from segment sums, so nothing becomes
  0/0; outputs stay finite and match the float64 definition.
* Records that leave the state unchanged: Mamba-2 dt = 0, GDN alpha = 1 with
  beta = 0.  The outputs are then those of the checkpoint alone.
* All-zero records from a zero state: outputs are exactly zero.
* A long run (1024 steps, 64 folds): float32 rounding does not accumulate.
* Corrupted pointer pairs (a negative count, a count above L, a negative pair)
  on a full window: a step, verify or flush stores nothing at all (ring,
  checkpoint and output byte-identical), leaves the pointers as they were and
  sets the status bit.
"""
import numpy as np
import pytest

from _gpu import announce, ckpt_rel_err, host, to_dev
from _metrics import max_rel_err
from oracle.session import StepwiseSession
from synth import InputStream, LayerShape

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _m2_layer(shape, A, D, S0, T=0):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    return ReplayLayer("mamba2", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       groups=shape.groups, max_draft=T, A=A, D=D, ckpt0=S0)


def _gdn_layer(shape, S0, T=0):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    return ReplayLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       max_draft=T, ckpt0=S0)


def _run(lay, ref, records, drafts_at=()):
    """Steps (and one verify + commit of all drafts where asked); every output finite and within TOL."""
    import torch
    worst = 0.0
    for t, r in enumerate(records):
        if t in drafts_at:
            d = {n: np.stack([a, a], axis=1) for n, a in r.items()}   # two drafts: the record twice
            y = host(lay.verify(to_dev(d)))
            assert np.all(np.isfinite(y))
            worst = max(worst, max_rel_err(y, ref.verify(d), ref.scale))
            acc = np.full(lay.shapes.batch, 2, np.int32)
            lay.commit(torch.from_numpy(acc).cuda())
            ref.commit(acc)
        else:
            y = host(lay.step(to_dev(r)))
            assert np.all(np.isfinite(y))
            worst = max(worst, max_rel_err(y, ref.step(r), ref.scale))
    assert worst <= TOL, worst
    lay.flush()
    assert ckpt_rel_err(host(lay.checkpoint), ref.state) <= TOL


def test_mamba2_decay_far_below_float32():
    shape = LayerShape("mamba2", 2, 8, 64, 128, 2, 16)
    announce("degenerate mamba2 fast decay", shape)
    ins = InputStream(shape, 51)
    A = np.full(shape.heads, -16.0, np.float32)
    A[::2] = -0.01                                    # slow heads next to the fast ones
    D = ins.params["D"]
    S0 = ins.initial_state(zeros=False, scale=0.5)
    recs = []
    for t in range(40):
        r = ins.record()
        r["dt"] = np.full_like(r["dt"], 8.0 if t % 5 else 0.5)
        recs.append(r)
    _run(_m2_layer(shape, A, D, S0, T=2), StepwiseSession("mamba2", S0, {"A": A, "D": D}), recs, drafts_at=(7, 23))


def test_mamba2_zero_dt_keeps_state():
    shape = LayerShape("mamba2", 2, 4, 64, 128, 2, 8)
    announce("degenerate mamba2 dt = 0", shape)
    ins = InputStream(shape, 52)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    recs = []
    for t in range(20):
        r = ins.record()
        if t % 3:
            r["dt"] = np.zeros_like(r["dt"])
        recs.append(r)
    _run(_m2_layer(shape, ins.params["A"], ins.params["D"], S0, T=2), StepwiseSession("mamba2", S0, ins.params),
         recs, drafts_at=(9,))


def test_gdn_decay_far_below_float32():
    shape = LayerShape("gdn", 2, 4, 128, 128, 4, 16)
    announce("degenerate gdn fast decay", shape)
    ins = InputStream(shape, 53)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    recs = []
    for t in range(40):
        r = ins.record()
        r["alpha"][:, ::2] = np.float32(1e-30)       # every other head forgets at once
        recs.append(r)
    _run(_gdn_layer(shape, S0, T=2), StepwiseSession("gdn", S0), recs, drafts_at=(5, 21))


def test_gdn_identity_records_keep_state():
    shape = LayerShape("gdn", 2, 4, 128, 128, 4, 8)
    announce("degenerate gdn alpha = 1, beta = 0", shape)
    ins = InputStream(shape, 54)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    recs = []
    for t in range(20):
        r = ins.record()
        if t % 2:
            r["alpha"] = np.ones_like(r["alpha"])
            r["beta"] = np.zeros_like(r["beta"])
        recs.append(r)
    _run(_gdn_layer(shape, S0, T=2), StepwiseSession("gdn", S0), recs, drafts_at=(11,))


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_zero_records_give_zero_outputs(kind):
    shape = LayerShape(kind, 2, 4, 64, 128, 2 if kind == "mamba2" else 4, 4)
    announce("degenerate zero records", shape)
    ins = InputStream(shape, 55)
    lay = _m2_layer(shape, ins.params["A"], ins.params["D"], None) if kind == "mamba2" else _gdn_layer(shape, None)
    for _ in range(9):                                # two folds
        r = {n: np.zeros_like(a) for n, a in ins.record().items()}
        if kind == "gdn":
            r["alpha"] = np.ones_like(r["alpha"])
        y = host(lay.step(to_dev(r)))
        assert np.all(y == 0.0)
    assert np.all(host(lay.checkpoint) == 0.0)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_long_run_stays_at_float32_rounding(kind):
    """1024 steps (64 folds) with verifies and commits every 50 steps: the float32
    checkpoint's rounding does not accumulate past the 1e-4 bar (the recurrence
    forgets at the synthetic decays)."""
    import torch
    shape = LayerShape(kind, 2, 8, 64, 128, 2 if kind == "mamba2" else 8, 16)
    announce("long run", shape)
    ins = InputStream(shape, 56)
    S0 = ins.initial_state(zeros=False, scale=0.5)
    if kind == "mamba2":
        lay = _m2_layer(shape, ins.params["A"], ins.params["D"], S0, T=4)
    else:
        lay = _gdn_layer(shape, S0, T=4)
    ref = StepwiseSession(kind, S0, ins.params)
    worst = 0.0
    for t in range(1024):
        if t % 50 == 49:
            d = ins.drafts(4)
            worst = max(worst, max_rel_err(host(lay.verify(to_dev(d))), ref.verify(d), ref.scale))
            acc = ins.accepted(4)
            lay.commit(torch.from_numpy(acc).cuda())
            ref.commit(acc)
        else:
            r = ins.record()
            worst = max(worst, max_rel_err(host(lay.step(to_dev(r))), ref.step(r), ref.scale))
    assert worst <= TOL, worst
    lay.flush()
    assert ckpt_rel_err(host(lay.checkpoint), ref.state) <= TOL


@pytest.mark.parametrize("in_ring", [False, True])
@pytest.mark.parametrize("call", ["step", "verify", "flush"])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_corrupted_pointers_store_nothing(kind, call, in_ring):
    """Three corrupted pointer pairs on a full window -- a negative count, a count
    above L, and a negative pair whose count (2) is in range -- for a step, a
    verify and a flush, with the records copied or in the ring: every sequence
    is flagged and skipped, so nothing is stored (ring, checkpoint and output
    byte-identical) and the pointers stay as they were."""
    import torch

    from _gpu import pointers_host
    from hybrid_model_ssm_replay_amd import binding as B
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    shape = LayerShape(kind, 3, 4, 32, 32, 2, 4) if kind == "mamba2" else LayerShape(kind, 3, 4, 64, 32, 4, 4)
    announce("corrupted pointers", shape, call, "in_ring", in_ring)
    ins = InputStream(shape, 8)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    kw = dict(groups=shape.groups, A=ins.params["A"], D=ins.params["D"]) if kind == "mamba2" else {}
    lay = ReplayLayer(kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      max_draft=2, ckpt0=S0, flags=B.FLAG_RECORDS_IN_RING if in_ring else 0, **kw)
    for _ in range(shape.window):  # full windows: a good next step would fold
        lay.step(to_dev(ins.record()))
    pos, ck = lay.pointers()
    pos[0] = ck[0] - 1                      # count -1 (a negative pos here: ck is 0)
    pos[1] = ck[1] + shape.window + 1       # count L + 1
    pos[2], ck[2] = -3, -5                  # count 2, both negative
    torch.cuda.synchronize()
    want_pos, want_ck = pointers_host(lay)
    ring0, ckpt0 = lay.ring.clone(), lay.ckpt.clone()
    if call == "step":
        y = torch.full((shape.batch, shape.heads, shape.head_dim), 7.0, device="cuda")
        lay.step(to_dev(ins.record()), y=y)
    elif call == "verify":
        y = torch.full((shape.batch, 2, shape.heads, shape.head_dim), 7.0, device="cuda")
        lay.verify(to_dev(ins.drafts(2)), y=y)
    else:
        y = None
        lay.flush()
    torch.cuda.synchronize()
    got_pos, got_ck = pointers_host(lay)
    assert lay.status & 0x2
    assert np.array_equal(got_pos, want_pos) and np.array_equal(got_ck, want_ck)
    assert torch.equal(lay.ring, ring0) and torch.equal(lay.ckpt, ckpt0)
    assert y is None or torch.all(y == 7.0)
