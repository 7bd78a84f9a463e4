"""Layer-level decode calls, built twice.  Test infrastructure only.

``StepwiseSession`` is the definition: it keeps the true state of every
sequence and advances it one token at a time (verify runs the drafts on a
copy; commit re-runs the accepted ones).

``ReplaySession`` is the method: a checkpoint plus the records since it,
driven by ``PointerMachine``; outputs come from the replay identities of
``mamba2`` / ``gdn`` and the checkpoint changes only at a fold.

Both expose init-time state and the calls step / verify / commit / flush with
the same argument shapes: a record is a dict of per-field arrays with a
leading batch axis; drafts have axes [batch, T, ...]; outputs are
[batch, H, head_dim] for a step and [batch, T, H, head_dim] for a verify.
The pages state that replay outputs equal conventional decoding up to
floating-point rounding [P2, paragraph 3; P3, Interpretation 2]; the tests
check exactly that between the two classes.
"""
from __future__ import annotations

import numpy as np

from . import gdn, mamba2
from .pointers import PointerMachine


def _rec_b(rec, b):
    return {n: a[b] for n, a in rec.items()}


def _draft_b(drafts, b, i):
    return {n: a[b, i] for n, a in drafts.items()}


class _Kind:
    """Per-family glue: stepwise update, replay output, fold."""

    def __init__(self, kind: str, params: dict):
        self.kind = kind
        self.params = {n: np.asarray(v, np.float64) for n, v in params.items()}

    def step(self, S, r):
        if self.kind == "mamba2":
            return mamba2.step(S, r["x"], r["B"], r["C"], r["dt"], self.params["A"], self.params["D"])
        return gdn.step(S, r["q"], r["k"], r["v"], r["alpha"], r["beta"])

    def output(self, S0, recs):
        if self.kind == "mamba2":
            return mamba2.replay_output(S0, recs, self.params["A"], self.params["D"])
        return gdn.replay_output(S0, recs, recs[-1]["q"])

    def fold(self, S0, recs):
        if self.kind == "mamba2":
            return mamba2.fold(S0, recs, self.params["A"])
        return gdn.fold(S0, recs)


class StepwiseSession:
    def __init__(self, kind: str, state0, params: dict | None = None):
        self.k = _Kind(kind, params or {})
        self.state = np.array(state0, np.float64)       # [batch, H, P, N]
        self.pending = None

    def step(self, rec):
        self.pending = None
        self.state, y = self.k.step(self.state, rec)
        return y

    def verify(self, drafts):
        T = next(iter(drafts.values())).shape[1]
        S = self.state.copy()
        ys = []
        for i in range(T):
            S, y = self.k.step(S, {n: a[:, i] for n, a in drafts.items()})
            ys.append(y)
        self.pending = drafts
        return np.stack(ys, axis=1)

    def commit(self, accepted):
        T = 0 if self.pending is None else next(iter(self.pending.values())).shape[1]
        for b, a in enumerate(np.asarray(accepted)):
            for i in range(int(np.clip(a, 0, T))):
                self.state[b], _ = self.k.step(self.state[b], _draft_b(self.pending, b, i))
        self.pending = None

    def flush(self, mask=None):
        pass                                            # the state is always exact


class ReplaySession:
    def __init__(self, kind: str, state0, window: int, params: dict | None = None):
        self.k = _Kind(kind, params or {})
        self.ckpt = np.array(state0, np.float64)        # [batch, H, P, N]
        self.ptr = PointerMachine(self.ckpt.shape[0], window)
        self.recs = [dict() for _ in range(self.ckpt.shape[0])]   # position -> record

    @property
    def batch(self):
        return self.ckpt.shape[0]

    def _window(self, b, upto):
        return [self.recs[b][p] for p in range(int(self.ptr.ckpt_pos[b]), upto)]

    def _fold(self, b):
        pos = int(self.ptr.pos[b])
        self.ckpt[b] = self.k.fold(self.ckpt[b], self._window(b, pos))
        for p in [p for p in self.recs[b] if p < pos]:
            del self.recs[b][p]                          # folded records leave the window

    def step(self, rec):
        will_fold = self.ptr.count == self.ptr.L
        for b in np.nonzero(will_fold)[0]:
            self._fold(b)
        pos_before = self.ptr.pos.copy()
        self.ptr.step()
        ys = []
        for b in range(self.batch):
            self.recs[b][int(pos_before[b])] = _rec_b(rec, b)
            ys.append(self.k.output(self.ckpt[b], self._window(b, int(self.ptr.pos[b]))))
        return np.stack(ys)

    def verify(self, drafts):
        T = next(iter(drafts.values())).shape[1]
        will_fold = self.ptr.count + T > self.ptr.L
        for b in np.nonzero(will_fold)[0]:
            self._fold(b)
        self.ptr.verify(T)
        out = []
        for b in range(self.batch):
            p0 = int(self.ptr.pos[b])
            for i in range(T):
                self.recs[b][p0 + i] = _draft_b(drafts, b, i)
            committed = self._window(b, p0)
            out.append(np.stack([self.k.output(self.ckpt[b], committed + [self.recs[b][p0 + j] for j in range(i + 1)])
                                 for i in range(T)]))
        return np.stack(out)

    def commit(self, accepted):
        return self.ptr.commit(accepted)

    def flush(self, mask=None):
        m = np.ones(self.batch, bool) if mask is None else np.asarray(mask, bool)
        for b in np.nonzero(m & (self.ptr.count > 0))[0]:
            self._fold(b)
        return self.ptr.flush(m)
