"""Algorithmic HBM bytes of each decode call: what the method itself must move.

Counts one read of every input byte the call needs and one write of every byte
it must leave behind; caching, re-reads and work the method avoids are not
counted.  Float32 throughout (4 bytes).  Per sequence, for one layer:

Mamba-2 (x per head, B and C per group, dt per head; a ring record holds x, B, dt):
  record_in  = (H P + 2 G N + H) 4        new token's x, B, C, dt
  ring_rec   = (H P + G N + H) 4          one buffered record (C is not kept)
  state      = H P N 4
  non-fold step at window position m:     read  state + (m - 1) ring_rec + record_in
                                          write ring_rec + y (H P 4)
  fold (lazy, at the step that finds L records):  read  + L ring_rec, write + state
Gated DeltaNet (q, k, v, alpha, beta per head; a ring record holds k, the
pseudo-value u (d_v), alpha, beta):
  record_in  = H (2 dk + dv + 2) 4, ring_rec = H (dk + dv + 2) 4, state = H dv dk 4
  (same structure).  With a separate read copy the ring also keeps v (H dv 4
  per record): written by every step, read back by the fold, which re-solves
  the pseudo-values from the checkpoint.
Conventional step: read state + record_in, write state + y.
With the records in the ring (zero-copy append) a step reads the same bytes but
appends only what it computes itself (GDN: the pseudo-value u; Mamba-2: nothing);
the producer's write of the record is the producer's output, not counted here.
With bf16 records (vec_bytes = 2) the record vector fields (Mamba-2 x, B, C;
GDN q, k, v) count 2 bytes in the inputs and in the ring; scalars, GDN
pseudo-values, outputs and the state stay 4.
Replay verify of T drafts after c committed records: read state + c ring_rec +
T record_in, write T ring_rec + T y (+ fold-first: L' ring_rec read, state written).
Snapshot verify: read state + T record_in, write T states + T y.

The checkpoint stream is read once per step and written once per window, against
once read and once written per step for the conventional kernel [P1,
Interpretation 2; P3, Interpretation 2].
"""
from __future__ import annotations

from dataclasses import dataclass

E = 4  # bytes per float32

# Bytes per state element of each storage format (F32, F16_SR, F8E4M3, F4E2M1_B16,
# F4E2M1_CS); the two-axis copy adds one exponent byte per state column.
FORMAT_BYTES = {0: 4.0, 1: 2.0, 2: 1.0, 3: 0.5 + 1.0 / 16, 4: 0.5 + 1.0 / 16}


def stored_state_bytes(l: "Layer", fmt: int) -> float:
    """Bytes of one sequence's stored state in `fmt`."""
    b = FORMAT_BYTES[fmt] * l.heads * l.head_dim * l.state_dim
    return b + (l.heads * l.state_dim if fmt == 4 else 0)


@dataclass(frozen=True)
class Layer:
    kind: str
    batch: int
    heads: int
    head_dim: int
    state_dim: int
    groups: int
    window: int
    vec_bytes: int = 4  # bytes per record vector element (4 float32, 2 bf16)

    @property
    def state(self) -> int:
        return self.heads * self.head_dim * self.state_dim * E

    @property
    def record_in(self) -> int:
        H, P, N, G, V = self.heads, self.head_dim, self.state_dim, self.groups, self.vec_bytes
        if self.kind == "mamba2":
            return (H * P + 2 * G * N) * V + H * E
        return H * (2 * N + P) * V + 2 * H * E

    @property
    def ring_rec(self) -> int:
        H, P, N, G, V = self.heads, self.head_dim, self.state_dim, self.groups, self.vec_bytes
        if self.kind == "mamba2":
            return (H * P + G * N) * V + H * E
        return H * N * V + H * P * E + 2 * H * E  # k, the pseudo-value u (float32), alpha, beta

    @property
    def y(self) -> int:
        return self.heads * self.head_dim * E

    def appended(self, in_ring: bool = False) -> int:
        """Bytes a step writes into the ring."""
        if not in_ring:
            return self.ring_rec
        return 0 if self.kind == "mamba2" else self.heads * self.head_dim * E


def replay_step_bytes(l: Layer, m: int, fold: bool, in_ring: bool = False) -> tuple[int, int]:
    """(read, write) bytes of one step for the whole batch; m = window records after the append."""
    rd = l.state + (m - 1) * l.ring_rec + l.record_in
    wr = l.appended(in_ring) + l.y
    if fold:
        rd += l.window * l.ring_rec
        wr += l.state
    return rd * l.batch, wr * l.batch


def replay_window_mean(l: Layer, in_ring: bool = False) -> tuple[float, float]:
    """Mean (read, write) bytes per step over a steady-state window of L steps.

    In steady state the step that finds the window full folds it and then
    starts the next window with m = 1; the other L - 1 steps have m = 2..L.
    """
    rd = wr = 0
    for m in range(1, l.window + 1):
        r, w = replay_step_bytes(l, m, fold=(m == 1), in_ring=in_ring)
        rd += r
        wr += w
    return rd / l.window, wr / l.window


def split_window_mean(l: Layer, ckpt_fmt: int, read_fmt: int) -> tuple[float, float]:
    """Window-mean (read, write) bytes per step with a stored checkpoint in ckpt_fmt
    and a read copy in read_fmt (the same copy when equal): non-fold steps read the
    read copy; a fold reads the checkpoint and writes both copies (Gated DeltaNet;
    a separate read copy adds the buffered values v; Mamba-2 keeps no extra field)."""
    ck, rd = stored_state_bytes(l, ckpt_fmt), stored_state_bytes(l, read_fmt)
    vrec = l.heads * l.head_dim * l.vec_bytes if (l.kind == "gdn" and read_fmt != ckpt_fmt) else 0
    rd_sum = wr_sum = 0.0
    for m in range(1, l.window + 1):
        fold = m == 1
        r = (ck if fold else rd) + (m - 1) * l.ring_rec + l.record_in
        w = l.ring_rec + vrec + l.y
        if fold:
            r += l.window * (l.ring_rec + vrec)
            w += ck + (rd if read_fmt != ckpt_fmt else 0.0)
        rd_sum += r * l.batch
        wr_sum += w * l.batch
    return rd_sum / l.window, wr_sum / l.window


def conventional_step_bytes(l: Layer) -> tuple[int, int]:
    return (l.state + l.record_in) * l.batch, (l.state + l.y) * l.batch


def replay_verify_bytes(l: Layer, T: int, committed: int, fold_first: bool) -> tuple[int, int]:
    rd = l.state + committed * l.ring_rec + T * l.record_in
    wr = T * l.ring_rec + T * l.y
    if fold_first:
        wr += l.state
    return rd * l.batch, wr * l.batch


def snapshot_verify_bytes(l: Layer, T: int) -> tuple[int, int]:
    return (l.state + T * l.record_in) * l.batch, (T * l.state + T * l.y) * l.batch


def verify_session_bytes(l: Layer, T: int, accepted: list, calls: int) -> tuple[float, float]:
    """Mean (read, write) model bytes per replay-verify launch over `calls`
    verify + commit rounds from empty windows, the accepted counts cycling
    through `accepted` (int arrays [batch]).  Per sequence, a verify folds first
    when its window cannot take T more records (count + T > L), and either way
    reads the count committed records once; the commit then appends
    min(a, T) records to what is left in the window."""
    import numpy as np
    count = np.zeros(l.batch, dtype=np.int64)
    rd = wr = 0.0
    for i in range(calls):
        fold = count + T > l.window
        rd += float(l.state * l.batch + count.sum() * l.ring_rec + T * l.record_in * l.batch)
        wr += float(T * (l.ring_rec + l.y) * l.batch + fold.sum() * l.state)
        a = np.minimum(np.asarray(accepted[i % len(accepted)], dtype=np.int64), T)
        count = np.where(fold, 0, count) + a
    return rd / calls, wr / calls
