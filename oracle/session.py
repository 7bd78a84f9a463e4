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
After a step or verify, ``scale`` ([batch, H] or [batch, T, H]) is the size
of the terms each output vector sums (``mamba2.output_scale``,
``gdn.output_scale``) for the state that output reads, the denominator floor
of the parity tests' relative error.
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

    def output(self, S0, recs, skip_below=None):
        if self.kind == "mamba2":
            return mamba2.replay_output(S0, recs, self.params["A"], self.params["D"], skip_below)
        return gdn.replay_output(S0, recs, recs[-1]["q"], skip_below)

    def fold(self, S0, recs, skip_below=None):
        if self.kind == "mamba2":
            return mamba2.fold(S0, recs, self.params["A"], skip_below)
        return gdn.fold(S0, recs, skip_below)

    def scale(self, S, r):
        """Output term size for the state S after record r (one sequence)."""
        if self.kind == "mamba2":
            return mamba2.output_scale(S, r["C"], self.params["D"], r["x"])
        return gdn.output_scale(S, r["q"])


class _Scales:
    """Lazily computed output scales: a list of (S0, window records) per output,
    the state being the fold of the window into S0."""

    def __init__(self, k, shape):
        self.k, self.shape, self.items = k, shape, []

    def add(self, S0, recs, skip_below=None):
        self.items.append((S0, list(recs), skip_below))

    def value(self):
        out = [self.k.scale(self.k.fold(S0, recs, sk), recs[-1]) for S0, recs, sk in self.items]
        return np.stack(out).reshape(self.shape + (-1,))


class StepwiseSession:
    def __init__(self, kind: str, state0, params: dict | None = None):
        self.k = _Kind(kind, params or {})
        self.state = np.array(state0, np.float64)       # [batch, H, P, N]
        self.pending = None
        self._outs = []                                 # (state, record) of each output of the last call

    @property
    def scale(self):
        """Output term sizes of the last call ([batch, H] or [batch, T, H]), computed on demand."""
        sc = [np.stack([self.k.scale(S[b], _rec_b(r, b)) for b in range(len(S))]) for S, r in self._outs]
        return sc[0] if self._lead_T is None else np.stack(sc, axis=1)

    def step(self, rec):
        self.pending = None
        self.state, y = self.k.step(self.state, rec)
        self._outs, self._lead_T = [(self.state, rec)], None
        return y

    def verify(self, drafts):
        T = next(iter(drafts.values())).shape[1]
        S = self.state.copy()
        ys, self._outs, self._lead_T = [], [], T
        for i in range(T):
            r = {n: a[:, i] for n, a in drafts.items()}
            S, y = self.k.step(S, r)
            ys.append(y)
            self._outs.append((S, r))
        self.pending = drafts
        return np.stack(ys, axis=1)

    def commit(self, accepted):
        T = 0 if self.pending is None else next(iter(self.pending.values())).shape[1]
        for b, a in enumerate(np.asarray(accepted)):
            for i in range(int(np.clip(a, 0, T))):
                self.state[b], _ = self.k.step(self.state[b], _draft_b(self.pending, b, i))
        self.pending = None

    def flush(self, mask=None):
        self.pending = None                             # the state is always exact; drafts are dropped


class ReplaySession:
    """The method: checkpoint + ring of the last L records, lazy folds.  With
    decay_skip, heads whose window decay is below 2^-24 drop the checkpoint
    term in outputs and folds (see oracle/mamba2.py, oracle/gdn.py)."""

    def __init__(self, kind: str, state0, window: int, params: dict | None = None, decay_skip: bool = False):
        self.k = _Kind(kind, params or {})
        self.skip = mamba2.DECAY_SKIP_LOG if decay_skip else None
        self.ckpt = np.array(state0, np.float64)        # [batch, H, P, N]
        self.ptr = PointerMachine(self.ckpt.shape[0], window)
        self.recs = [dict() for _ in range(self.ckpt.shape[0])]   # position -> record
        self._scales = None

    @property
    def scale(self):
        return self._scales.value()

    @property
    def batch(self):
        return self.ckpt.shape[0]

    def _window(self, b, upto):
        return [self.recs[b][p] for p in range(int(self.ptr.ckpt_pos[b]), upto)]

    def _fold(self, b):
        pos = int(self.ptr.pos[b])
        self.ckpt[b] = self.k.fold(self.ckpt[b], self._window(b, pos), self.skip)
        for p in [p for p in self.recs[b] if p < pos]:
            del self.recs[b][p]                          # folded records leave the window

    def step(self, rec):
        will_fold = self.ptr.count == self.ptr.L
        for b in np.nonzero(will_fold)[0]:
            self._fold(b)
        pos_before = self.ptr.pos.copy()
        self.ptr.step()
        ys = []
        self._scales = _Scales(self.k, (self.batch,))
        for b in range(self.batch):
            self.recs[b][int(pos_before[b])] = _rec_b(rec, b)
            win = self._window(b, int(self.ptr.pos[b]))
            ys.append(self.k.output(self.ckpt[b], win, self.skip))
            self._scales.add(self.ckpt[b], win, self.skip)
        return np.stack(ys)

    def verify(self, drafts):
        T = next(iter(drafts.values())).shape[1]
        will_fold = self.ptr.count + T > self.ptr.L
        for b in np.nonzero(will_fold)[0]:
            self._fold(b)
        self.ptr.verify(T)
        out = []
        self._scales = _Scales(self.k, (self.batch, T))
        for b in range(self.batch):
            p0 = int(self.ptr.pos[b])
            for i in range(T):
                self.recs[b][p0 + i] = _draft_b(drafts, b, i)
            committed = self._window(b, p0)
            wins = [committed + [self.recs[b][p0 + j] for j in range(i + 1)] for i in range(T)]
            out.append(np.stack([self.k.output(self.ckpt[b], w, self.skip) for w in wins]))
            for w in wins:
                self._scales.add(self.ckpt[b], w, self.skip)
        return np.stack(out)

    def commit(self, accepted):
        return self.ptr.commit(accepted)

    def flush(self, mask=None):
        m = np.ones(self.batch, bool) if mask is None else np.asarray(mask, bool)
        for b in np.nonzero(m & (self.ptr.count > 0))[0]:
            self._fold(b)
        return self.ptr.flush(m)


# ---- split-precision state ---------------------------------------------------------
FMT_F32, FMT_F16_SR, FMT_F8E4M3, FMT_F4E2M1_B16, FMT_F4E2M1_CS = 0, 1, 2, 3, 4


def encode_state(S32, fmt, seed=0, b=0, ckpt_pos=0):
    """Stored form of one sequence's float32 state [H, P, N] in `fmt`."""
    from . import quant
    S32 = np.asarray(S32, np.float32)
    if fmt == FMT_F32:
        return S32.copy()
    if fmt == FMT_F16_SR:
        H = S32.shape[0]
        out = np.empty(S32.shape, np.float16)
        for h in range(H):
            r = quant.sr_bits(seed, b, h, ckpt_pos, S32[h].size).reshape(S32[h].shape)
            out[h] = quant.fp16_sr(S32[h], r)
        return out
    if fmt == FMT_F8E4M3:
        return quant.e4m3_encode(S32)
    if fmt == FMT_F4E2M1_B16:
        return quant.e2m1_block_encode(S32)
    if fmt == FMT_F4E2M1_CS:
        return quant.e2m1_cs_encode(S32)
    raise ValueError(fmt)


def decode_state(stored, fmt):
    from . import quant
    if fmt == FMT_F32:
        return np.asarray(stored, np.float64)
    if fmt == FMT_F16_SR:
        return np.asarray(stored, np.float64)
    if fmt == FMT_F8E4M3:
        return quant.e4m3_decode(stored).astype(np.float64)
    if fmt == FMT_F4E2M1_CS:
        return quant.e2m1_cs_decode(*stored)
    return quant.e2m1_block_decode(*stored).astype(np.float64)


class SplitReplaySession(ReplaySession):
    """Replay with the checkpoint stored in ckpt_fmt (it carries the recurrence)
    and a read copy in read_fmt; read_fmt == ckpt_fmt is one shared copy.  The
    pages separate the two precisions so that the read copy's rounding never
    re-enters the recurrence [P1, Interpretation 4; P3, Interpretation 3], and
    say that the outputs of steps that do not fold still depend on the
    approximate copy [P3, Perspective, paragraph 2]; the call that folds holds
    the exact fold result.  Readings:

    * a fold starts from the decoded recurrence copy, folds in full precision,
      rounds to float32 and encodes both copies from that float32 state;
    * the outputs of a step or verify that folds first come from the fold
      result itself (full precision), with the call's records;
    * every other output comes from the decoded read copy plus the buffered
      records (which are exact), so within a window the pseudo-values of the
      Gated DeltaNet form are those of the read copy, also for the record the
      fold step appended.
    """

    def __init__(self, kind, state0, window, params=None, ckpt_fmt=FMT_F32, read_fmt=FMT_F32, seed=0):
        super().__init__(kind, state0, window, params)
        self.cf, self.rf, self.seed = ckpt_fmt, read_fmt, seed
        S32 = np.asarray(state0, np.float32)
        B = S32.shape[0]
        self.R = [encode_state(S32[b], ckpt_fmt, seed, b, 0) for b in range(B)]
        self.Q = self.R if read_fmt == ckpt_fmt else [encode_state(S32[b], read_fmt, seed, b, 0) for b in range(B)]
        self.last_fold = {}                             # b -> float64 fold result of the latest fold

    def read_state(self, b):
        return decode_state(self.Q[b], self.rf)

    def recurrence_state(self, b):
        return decode_state(self.R[b], self.cf)

    def _fold(self, b):
        pos = int(self.ptr.pos[b])
        S = self.k.fold(self.recurrence_state(b), self._window(b, pos))
        S32 = S.astype(np.float32)
        self.R[b] = encode_state(S32, self.cf, self.seed, b, pos)
        if self.Q is not self.R:
            self.Q[b] = encode_state(S32, self.rf, self.seed, b, pos)
        self.last_fold[b] = S
        for p in [p for p in self.recs[b] if p < pos]:
            del self.recs[b][p]
        return S

    def step(self, rec):
        will_fold = self.ptr.count == self.ptr.L
        fresh = {int(b): self._fold(b) for b in np.nonzero(will_fold)[0]}
        pos_before = self.ptr.pos.copy()
        self.ptr.step()
        ys = []
        self._scales = _Scales(self.k, (self.batch,))
        for b in range(self.batch):
            self.recs[b][int(pos_before[b])] = _rec_b(rec, b)
            S0 = fresh[b] if b in fresh else self.read_state(b)
            win = self._window(b, int(self.ptr.pos[b]))
            ys.append(self.k.output(S0, win))
            self._scales.add(S0, win)
        return np.stack(ys)

    def verify(self, drafts):
        T = next(iter(drafts.values())).shape[1]
        will_fold = self.ptr.count + T > self.ptr.L
        fresh = {int(b): self._fold(b) for b in np.nonzero(will_fold)[0]}
        self.ptr.verify(T)
        out = []
        self._scales = _Scales(self.k, (self.batch, T))
        for b in range(self.batch):
            p0 = int(self.ptr.pos[b])
            for i in range(T):
                self.recs[b][p0 + i] = _draft_b(drafts, b, i)
            committed = self._window(b, p0)
            S0 = fresh[b] if b in fresh else self.read_state(b)
            wins = [committed + [self.recs[b][p0 + j] for j in range(i + 1)] for i in range(T)]
            out.append(np.stack([self.k.output(S0, w) for w in wins]))
            for w in wins:
                self._scales.add(S0, w)
        return np.stack(out)

    def flush(self, mask=None):
        m = np.ones(self.batch, bool) if mask is None else np.asarray(mask, bool)
        for b in np.nonzero(m & (self.ptr.count > 0))[0]:
            self._fold(b)
        return self.ptr.flush(m)
