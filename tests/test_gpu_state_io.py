"""Checkpoint / resume and determinism on the GPU.

The checkpoint of this method is the layer state itself: after an explicit
flush a sequence's whole state is its stored checkpoint (and read copy), plus
its pointers; the window is empty.  Saving it is a copy of those buffers, and
resuming from it (in the same layer or a fresh one) must continue exactly as
an uninterrupted run: bit-identical outputs and stored bytes.

Determinism: each (sequence, head) tile is computed by one workgroup with no
atomics on data, and stochastic rounding draws counter-based bits (Philox
keyed by position), so two runs of the same calls give identical bytes.
"""
import numpy as np
import pytest

from _gpu import announce, to_dev
from synth import InputStream, LayerShape

pytestmark = pytest.mark.gpu
SEED = 0x5EED


def _layer(shape, ins, cf=0, rf=0, max_draft=0, S0=None):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    kw = dict(A=ins.params["A"], D=ins.params["D"], groups=shape.groups) if shape.kind == "mamba2" else {}
    return ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                       max_draft=max_draft, ckpt_fmt=cf, read_fmt=rf, seed=SEED, ckpt0=S0, **kw)


def _save(lay):
    """The state after a flush: stored copies and the current pointers."""
    import torch
    torch.cuda.synchronize()
    ck, rd = lay.stored_copies()
    pos, ckp = lay.pointers()
    return (ck.clone(), None if rd is None else rd.clone(), pos.clone(), ckp.clone())


def _restore(lay, saved):
    import torch
    ck, rd = lay.stored_copies()
    ck.copy_(saved[0])
    if rd is not None:
        rd.copy_(saved[1])
    pos, ckp = lay.pointers()
    pos.copy_(saved[2])
    ckp.copy_(saved[3])
    torch.cuda.synchronize()


def _continue(lay, ins, n, T):
    """n calls on a copy of the input stream ins (ins itself does not advance):
    steps, with a verify + commit every third call."""
    import copy

    import torch
    ins = copy.deepcopy(ins)
    outs = []
    for i in range(n):
        if i % 3 == 2:
            d = ins.drafts(T)
            outs.append(lay.verify(to_dev(d)).clone())
            lay.commit(torch.from_numpy(ins.accepted(T)).cuda())
        else:
            outs.append(lay.step(to_dev(ins.record())).clone())
    torch.cuda.synchronize()
    return [o.cpu() for o in outs]


CASES = [("mamba2", 0, 0), ("mamba2", 0, 3), ("mamba2", 1, 3), ("gdn", 0, 0), ("gdn", 0, 3), ("gdn", 1, 3), ("gdn", 3, 3)]


@pytest.mark.parametrize("kind,cf,rf", CASES)
def test_flush_save_resume_is_bit_exact(kind, cf, rf):
    import torch
    shape = (LayerShape("mamba2", 3, 4, 64, 128, 2, 4) if kind == "mamba2"
             else LayerShape("gdn", 3, 4, 128, 128, 4, 4))
    announce("checkpoint/resume", shape, cf, rf)
    ins = InputStream(shape, 40)
    S0 = ins.initial_state(zeros=False, scale=0.3)
    lay = _layer(shape, ins, cf, rf, max_draft=3, S0=S0)
    for _ in range(6):                                   # one fold and part of a window
        lay.step(to_dev(ins.record()))
    lay.flush()
    saved = _save(lay)
    first = _continue(lay, ins, 11, 3)                # uninterrupted run from the flush
    end_bytes = [t.clone() for t in lay.stored_copies() if t is not None]
    _restore(lay, saved)                                 # resume in the same layer
    again = _continue(lay, ins, 11, 3)
    fresh = _layer(shape, ins, cf, rf, max_draft=3)      # resume in a new layer
    _restore(fresh, saved)
    other = _continue(fresh, ins, 11, 3)
    for a, b, c in zip(first, again, other):
        assert torch.equal(a, b) and torch.equal(a, c)
    for t0, t1, t2 in zip(end_bytes, [t for t in lay.stored_copies() if t is not None],
                          [t for t in fresh.stored_copies() if t is not None]):
        assert torch.equal(t0, t1) and torch.equal(t0, t2)
    assert lay.status == 0 and fresh.status == 0


@pytest.mark.parametrize("kind,cf,rf", CASES + [("gdn", 2, 4)])
def test_runs_are_deterministic(kind, cf, rf):
    """Steps through folds, verifies with fold-firsts and commits, twice from the
    same inputs: identical outputs and stored bytes (stochastic rounding included)."""
    import torch
    shape = (LayerShape("mamba2", 2, 8, 64, 128, 2, 4) if kind == "mamba2"
             else LayerShape("gdn", 2, 8, 128, 128, 8, 4))
    announce("determinism", shape, cf, rf)
    runs = []
    for _ in range(2):
        ins = InputStream(shape, 41)
        lay = _layer(shape, ins, cf, rf, max_draft=3, S0=ins.initial_state(zeros=False, scale=0.3))
        outs = _continue(lay, ins, 14, 3)
        runs.append((outs, [t.clone().cpu() for t in lay.stored_copies() if t is not None], lay.ring.clone().cpu()))
    for a, b in zip(runs[0][0], runs[1][0]):
        assert torch.equal(a, b)
    for a, b in zip(runs[0][1], runs[1][1]):
        assert torch.equal(a, b)
    assert torch.equal(runs[0][2], runs[1][2])
