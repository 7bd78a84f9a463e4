"""Buffer-pointer machine of the replay decode path.  Test infrastructure only.

Integers only.  Per sequence: ``pos`` (tokens committed so far), ``ckpt_pos``
(tokens folded into the checkpoint); the window holds the records at
positions ckpt_pos .. pos-1, so count = pos - ckpt_pos is always in 0..L.
Drafts of a pending verify sit at positions pos .. pos+T-1.

Rules (the pages state the behaviour; the exact flush timing is a reading):

* step: if the window is full (count == L) it is folded first
  (ckpt_pos = pos); then the new record is appended at position pos and pos
  advances by one.  The checkpoint is therefore written only when the buffer
  has filled, once per L tokens without speculation [P2, paragraph 3;
  P3, Interpretation 2].  Folding lazily, at the step that finds the window
  full, is the reading taken where the pages leave the moment open.
* verify(T), 1 <= T <= L: if count + T > L the committed records are folded
  first; the T drafts then go to positions pos .. pos+T-1; nothing else moves.
  Verification produces outputs only and writes no intermediate state
  [P1, Interpretation 3; P3, Interpretation 3].
* commit(a): pos += min(max(a, 0), T_pending); rollback of rejected drafts is
  just not advancing the pointer [P1, Interpretation 3; P3, Interpretation 3].
  An out-of-range a is clamped and flagged.
* A step, verify or flush issued while drafts are pending discards them (the
  same as commit(0)); only commit consumes them.
* flush(mask): fold every committed record of the masked sequences
  (ckpt_pos = pos); sequences with an empty window are left alone.
"""
from __future__ import annotations

import numpy as np

STATUS_ACCEPT_CLAMPED = 0x1


class PointerMachine:
    def __init__(self, batch: int, window: int):
        if not 1 <= window <= 16:
            raise ValueError("window must be in 1..16")
        self.L = window
        self.pos = np.zeros(batch, np.int64)
        self.ckpt_pos = np.zeros(batch, np.int64)
        self.t_pending = 0
        self.status = 0

    @property
    def count(self) -> np.ndarray:
        return self.pos - self.ckpt_pos

    def step(self) -> np.ndarray:
        """Advance one token.  Returns the mask of sequences folded first."""
        self.t_pending = 0
        folded = self.count == self.L
        self.ckpt_pos = np.where(folded, self.pos, self.ckpt_pos)
        self.pos = self.pos + 1
        return folded

    def verify(self, T: int) -> np.ndarray:
        """Stage T drafts.  Returns the mask of sequences folded first."""
        if not 1 <= T <= self.L:
            raise ValueError("draft count must be in 1..L")
        folded = self.count + T > self.L
        self.ckpt_pos = np.where(folded, self.pos, self.ckpt_pos)
        self.t_pending = T
        return folded

    def commit(self, accepted) -> np.ndarray:
        """Advance by the accepted prefix.  Returns the per-sequence advance."""
        a = np.asarray(accepted, np.int64)
        adv = np.clip(a, 0, self.t_pending)
        if np.any(adv != a):
            self.status |= STATUS_ACCEPT_CLAMPED
        self.pos = self.pos + adv
        self.t_pending = 0
        return adv

    def flush(self, mask=None) -> np.ndarray:
        """Fold the committed window of masked sequences.  Returns who folded."""
        m = np.ones_like(self.pos, bool) if mask is None else np.asarray(mask, bool)
        folded = m & (self.count > 0)
        self.ckpt_pos = np.where(folded, self.pos, self.ckpt_pos)
        self.t_pending = 0
        return folded
