"""Pins for the buffer-pointer machine: a hand-worked trace and invariants."""
import os

import numpy as np
import pytest

from oracle.pointers import STATUS_ACCEPT_CLAMPED, PointerMachine

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pointer_trace_L4.txt")


def _load_trace():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lhs, rhs = line.split("|")
        op, arg = lhs.split()
        rows.append((op, None if arg == "-" else int(arg), tuple(int(v) for v in rhs.split())))
    return rows


def test_hand_worked_trace():
    pm = PointerMachine(1, 4)
    rows = _load_trace()
    assert len(rows) == 26
    for op, arg, (pos, ckpt, folded, status) in rows:
        if op == "step":
            f = pm.step()[0]
        elif op == "verify":
            f = pm.verify(arg)[0]
        elif op == "commit":
            pm.commit([arg]); f = False
        else:
            f = pm.flush()[0]
        assert (int(pm.pos[0]), int(pm.ckpt_pos[0]), int(f), pm.status) == (pos, ckpt, folded, status), (op, arg)


@pytest.mark.parametrize("L", [1, 4, 16])
def test_plain_decoding_folds_once_per_window(L):
    # Without speculation the checkpoint is written once every L tokens: after
    # n steps, exactly floor((n - 1) / L) folds have happened.
    pm = PointerMachine(3, L)
    folds = 0
    for n in range(1, 5 * L + 3):
        folds += int(pm.step()[0])
        assert folds == (n - 1) // L
        assert np.all(pm.count >= 1) and np.all(pm.count <= L)


def test_random_ops_keep_invariants():
    rng = np.random.default_rng(0)
    for L in (1, 2, 5, 16):
        pm = PointerMachine(8, L)
        last_pos = pm.pos.copy()
        for _ in range(400):
            op = rng.integers(4)
            if op == 0:
                pm.step()
            elif op == 1:
                T = int(rng.integers(1, L + 1))
                pm.verify(T)
                assert np.all(pm.count + T <= L)
                pm.commit(rng.integers(0, T + 1, size=8))
            elif op == 2:
                pm.flush(rng.integers(0, 2, size=8).astype(bool))
            else:
                pm.commit(np.zeros(8, int))               # no pending drafts: a no-op
            assert np.all(pm.pos >= last_pos)
            assert np.all((pm.count >= 0) & (pm.count <= L))
            last_pos = pm.pos.copy()
        assert pm.status == 0


def test_commit_zero_is_noop_and_clamp_flags():
    pm = PointerMachine(2, 8)
    pm.step(); pm.step()
    pm.verify(3)
    before = (pm.pos.copy(), pm.ckpt_pos.copy())
    pm.commit([0, 0])
    assert np.array_equal(pm.pos, before[0]) and np.array_equal(pm.ckpt_pos, before[1])
    assert pm.status == 0
    pm.verify(3)
    pm.commit([7, -1])
    assert list(pm.pos) == [5, 2] and pm.status == STATUS_ACCEPT_CLAMPED


def test_rejects_bad_draft_count():
    pm = PointerMachine(1, 4)
    with pytest.raises(ValueError):
        pm.verify(5)
    with pytest.raises(ValueError):
        pm.verify(0)


def test_flush_discards_pending_drafts():
    # Only a commit consumes pending drafts; a flush between a verify and its
    # commit drops them (as a step or a verify would), so the commit clamps.
    pm = PointerMachine(2, 8)
    pm.step(); pm.step()
    pm.verify(3)
    folded = pm.flush(np.array([True, False]))
    assert list(folded) == [True, False] and list(pm.ckpt_pos) == [2, 0]
    pm.commit([2, 0])
    assert list(pm.pos) == [2, 2] and pm.status == STATUS_ACCEPT_CLAMPED
