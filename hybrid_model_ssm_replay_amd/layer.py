"""PyTorch-owned device buffers around the C calls.

``ReplayLayer`` allocates the checkpoint, ring, pointer words and status word of
one layer with torch, fills a ``replay_ctx`` through ``replay_init`` and then
forwards step / verify / commit / flush to the library on the current stream.
``ConvLayer`` and ``SnapshotLayer`` do the same for the two in-run baselines.
No arithmetic of the decode path happens here.
"""
from __future__ import annotations

import torch

from . import binding as B

_FIELDS = {B.KIND_MAMBA2: ("x", "B", "C", "dt"), B.KIND_GDN: ("q", "k", "v", "alpha", "beta")}
_VECTOR_FIELDS = ("x", "B", "C", "q", "k", "v")  # bf16 with FLAG_BF16_RECORDS; the scalars stay float32
# Fields the ring keeps, written by the producer with FLAG_RECORDS_IN_RING (record field index).
RING_FIELDS = {B.KIND_MAMBA2: {"x": 0, "B": 1, "dt": 3}, B.KIND_GDN: {"k": 1, "alpha": 3, "beta": 4}}


def _kind(kind) -> int:
    if kind in (B.KIND_MAMBA2, "mamba2"):
        return B.KIND_MAMBA2
    if kind in (B.KIND_GDN, "gdn"):
        return B.KIND_GDN
    raise ValueError(f"unknown kind {kind!r}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev_f32(t: torch.Tensor, shape, name, dtype=torch.float32) -> torch.Tensor:
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


class _Shapes:
    def __init__(self, kind, batch, heads, groups, head_dim, state_dim, flags=0):
        self.kind, self.batch, self.heads, self.groups = kind, batch, heads, groups
        self.head_dim, self.state_dim = head_dim, state_dim
        self.vec_dtype = torch.bfloat16 if flags & B.FLAG_BF16_RECORDS else torch.float32
        self.in_ring = bool(flags & B.FLAG_RECORDS_IN_RING)

    def field_shapes(self, lead):
        H, G, P, N = self.heads, self.groups, self.head_dim, self.state_dim
        if self.kind == B.KIND_MAMBA2:
            return {"x": lead + (H, P), "B": lead + (G, N), "C": lead + (G, N), "dt": lead + (H,)}
        return {"q": lead + (H, N), "k": lead + (H, N), "v": lead + (H, P), "alpha": lead + (H,),
                "beta": lead + (H,)}

    def record(self, fields: dict, lead, use_ring=False) -> tuple[B.replay_record, list]:
        """The record struct of `fields`; with use_ring the fields the ring keeps
        are not passed (the producer wrote them into their ring slots)."""
        shapes = self.field_shapes(lead)
        skip = RING_FIELDS[self.kind] if use_ring else {}
        keep = [None if n in skip else
                _dev_f32(fields[n], shapes[n], n, self.vec_dtype if n in _VECTOR_FIELDS else torch.float32)
                for n in _FIELDS[self.kind]]
        return B.make_record(*[0 if t is None else t.data_ptr() for t in keep]), keep


class ReplayLayer:
    """One layer's replay state on the current CUDA (HIP) device."""

    def __init__(self, kind, batch, heads, head_dim, state_dim, window, groups=None, max_draft=0,
                 ckpt_fmt=B.FMT_F32, read_fmt=B.FMT_F32, seed=0, A=None, D=None, ckpt0=None, device="cuda",
                 flags=0):
        B.load_library()
        k = _kind(kind)
        groups = heads if groups is None else groups
        self.shapes = _Shapes(k, batch, heads, groups, head_dim, state_dim, flags)
        self.cfg = B.make_config(k, batch, heads, groups, head_dim, state_dim, window, max_draft, ckpt_fmt,
                                 read_fmt, seed, flags)
        rc = B.replay_validate_config(self.cfg)
        if rc != B.OK:
            raise B.ReplayError("replay_validate_config", rc)
        dev = torch.device(device)
        self.ckpt = torch.zeros(B.replay_ckpt_bytes(self.cfg), dtype=torch.uint8, device=dev)
        if ckpt0 is not None and ckpt_fmt == B.FMT_F32:
            self.ckpt.view(torch.float32).copy_(torch.as_tensor(ckpt0, dtype=torch.float32).reshape(-1))
        rc_bytes = B.replay_read_copy_bytes(self.cfg)
        self.read_copy = torch.zeros(max(rc_bytes, 16), dtype=torch.uint8, device=dev) if rc_bytes else None
        self.ring = torch.zeros(B.replay_ring_bytes(self.cfg), dtype=torch.uint8, device=dev)
        self.pointer_words = torch.zeros(B.replay_pointer_words(self.cfg), dtype=torch.int32, device=dev)
        self.status_word = torch.zeros(4, dtype=torch.int32, device=dev)
        if k == B.KIND_MAMBA2:
            if A is None or D is None:
                raise ValueError("Mamba-2 needs A and D")
            self.A = torch.as_tensor(A, dtype=torch.float32).to(dev).contiguous()
            self.D = torch.as_tensor(D, dtype=torch.float32).to(dev).contiguous()
            _dev_f32(self.A, (heads,), "A")
            _dev_f32(self.D, (heads,), "D")
        else:
            self.A = self.D = None
        self.buf = B.replay_buffers(self.ckpt.data_ptr(), self.read_copy.data_ptr() if self.read_copy is not None
                                    else None, self.ring.data_ptr(), self.pointer_words.data_ptr(),
                                    self.status_word.data_ptr(), self.A.data_ptr() if self.A is not None else None,
                                    self.D.data_ptr() if self.D is not None else None)
        self.ctx = B.replay_ctx()
        B.replay_init(self.ctx, self.cfg, self.buf, _stream())
        if ckpt0 is not None and ckpt_fmt != B.FMT_F32:
            self.set_state(torch.as_tensor(ckpt0, dtype=torch.float32).to(dev))

    # -- views ---------------------------------------------------------------
    @property
    def checkpoint(self) -> torch.Tensor:
        """The float32 checkpoint (F32 checkpoint format only)."""
        if self.cfg.ckpt_fmt != B.FMT_F32:
            raise ValueError("the checkpoint is stored in a low-precision format; see stored_copies()")
        s = self.shapes
        return self.ckpt.view(torch.float32).view(s.batch, s.heads, s.head_dim, s.state_dim)

    def stored_copies(self):
        """Raw device bytes of (checkpoint, read copy or None), in their formats."""
        return self.ckpt, self.read_copy

    def set_state(self, state: torch.Tensor) -> None:
        s = self.shapes
        st = _dev_f32(state.contiguous(), (s.batch, s.heads, s.head_dim, s.state_dim), "state")
        B.replay_set_state(self.ctx, st.data_ptr(), _stream())

    def pointers(self) -> tuple[torch.Tensor, torch.Tensor]:
        """(pos, ckpt_pos) device views of the current pointer half."""
        pos_addr, ck_addr = B.replay_current_pointers(self.ctx)
        base = self.pointer_words.data_ptr()
        Bt = self.shapes.batch
        i0, i1 = (pos_addr - base) // 4, (ck_addr - base) // 4
        return self.pointer_words[i0:i0 + Bt], self.pointer_words[i1:i1 + Bt]

    @property
    def status(self) -> int:
        return int(self.status_word[0].item())

    @property
    def t_pending(self) -> int:
        return int(self.ctx.t_pending)

    # -- calls ---------------------------------------------------------------
    def _out(self, lead):
        s = self.shapes
        return torch.empty(lead + (s.heads, s.head_dim), dtype=torch.float32, device=self.ckpt.device)

    def ring_fields(self) -> dict:
        """Device views of the ring fields a producer writes (FLAG_RECORDS_IN_RING):
        Mamba-2 x [slots][B][H][P], B [B][G][slots][N], dt [B][H][slots];
        GDN k [slots][B][H][dk], alpha and beta [B][H][slots]."""
        view = B.replay_ring_fields(self.ctx)
        s, n = self.shapes, view.slots
        base = self.ring.data_ptr()
        vec_size = 2 if s.vec_dtype == torch.bfloat16 else 4

        def at(addr, dtype, shape, esize):
            off = addr - base
            numel = 1
            for d in shape:
                numel *= d
            return self.ring[off:off + numel * esize].view(dtype).view(shape)

        if s.kind == B.KIND_MAMBA2:
            return {"x": at(view.f[0], s.vec_dtype, (n, s.batch, s.heads, s.head_dim), vec_size),
                    "B": at(view.f[1], s.vec_dtype, (s.batch, s.groups, n, s.state_dim), vec_size),
                    "dt": at(view.f[3], torch.float32, (s.batch, s.heads, n), 4)}
        return {"k": at(view.f[1], s.vec_dtype, (n, s.batch, s.heads, s.state_dim), vec_size),
                "alpha": at(view.f[3], torch.float32, (s.batch, s.heads, n), 4),
                "beta": at(view.f[4], torch.float32, (s.batch, s.heads, n), 4)}

    def record_slots(self) -> torch.Tensor:
        """Ring slot of each sequence's next record (int32 [batch], FLAG_RECORDS_IN_RING)."""
        out = torch.empty(self.shapes.batch, dtype=torch.int32, device=self.ckpt.device)
        B.replay_record_slots(self.ctx, out.data_ptr(), _stream())
        return out

    def step(self, rec: dict, y: torch.Tensor | None = None) -> torch.Tensor:
        lead = (self.shapes.batch,)
        r, keep = self.shapes.record(rec, lead, self.shapes.in_ring)
        y = self._out(lead) if y is None else _dev_f32(y, lead + (self.shapes.heads, self.shapes.head_dim), "y")
        B.replay_step(self.ctx, r, y.data_ptr(), _stream())
        return y

    def verify(self, drafts: dict, y: torch.Tensor | None = None) -> torch.Tensor:
        T = int(next(iter(drafts.values())).shape[1])
        lead = (self.shapes.batch, T)
        r, keep = self.shapes.record(drafts, lead, self.shapes.in_ring)
        y = self._out(lead) if y is None else _dev_f32(y, lead + (self.shapes.heads, self.shapes.head_dim), "y")
        B.replay_verify(self.ctx, T, r, y.data_ptr(), _stream())
        return y

    def commit(self, accepted: torch.Tensor) -> None:
        if not (accepted.is_cuda and accepted.dtype == torch.int32 and accepted.is_contiguous()
                and tuple(accepted.shape) == (self.shapes.batch,)):
            raise ValueError("accepted must be a contiguous int32 device tensor [batch]")
        B.replay_commit(self.ctx, accepted.data_ptr(), _stream())

    def flush(self, mask: torch.Tensor | None = None) -> None:
        if mask is not None and not (mask.is_cuda and mask.dtype == torch.uint8 and mask.is_contiguous()
                                     and tuple(mask.shape) == (self.shapes.batch,)):
            raise ValueError("mask must be a contiguous uint8 device tensor [batch]")
        B.replay_flush(self.ctx, mask.data_ptr() if mask is not None else None, _stream())


class ConvLayer:
    """Baseline: conventional load-update-store decode step on an F32 state."""

    def __init__(self, kind, batch, heads, head_dim, state_dim, groups=None, A=None, D=None, state0=None,
                 device="cuda", flags=0):
        B.load_library()
        k = _kind(kind)
        groups = heads if groups is None else groups
        self.shapes = _Shapes(k, batch, heads, groups, head_dim, state_dim, flags)
        self.cfg = B.make_config(k, batch, heads, groups, head_dim, state_dim, 1, 0, flags=flags)
        dev = torch.device(device)
        self.state = torch.zeros((batch, heads, head_dim, state_dim), dtype=torch.float32, device=dev)
        if state0 is not None:
            self.state.copy_(torch.as_tensor(state0, dtype=torch.float32))
        self.A = torch.as_tensor(A, dtype=torch.float32).to(dev).contiguous() if A is not None else None
        self.D = torch.as_tensor(D, dtype=torch.float32).to(dev).contiguous() if D is not None else None

    def step(self, rec: dict, y: torch.Tensor | None = None) -> torch.Tensor:
        s = self.shapes
        r, keep = s.record(rec, (s.batch,))
        if y is None:
            y = torch.empty((s.batch, s.heads, s.head_dim), dtype=torch.float32, device=self.state.device)
        B.replay_conv_step(self.cfg, self.state.data_ptr(), self.A.data_ptr() if self.A is not None else 0,
                           self.D.data_ptr() if self.D is not None else 0, r, y.data_ptr(), _stream())
        return y


class SnapshotLayer:
    """Baseline: verification that stores one state snapshot per draft token."""

    def __init__(self, kind, batch, heads, head_dim, state_dim, max_draft, groups=None, A=None, D=None,
                 state0=None, device="cuda", flags=0):
        B.load_library()
        k = _kind(kind)
        groups = heads if groups is None else groups
        self.shapes = _Shapes(k, batch, heads, groups, head_dim, state_dim, flags)
        self.cfg = B.make_config(k, batch, heads, groups, head_dim, state_dim, max(max_draft, 1), max_draft,
                                 flags=flags)
        dev = torch.device(device)
        self.nslots = max_draft + 1
        self.slots = torch.zeros((batch, self.nslots, heads, head_dim, state_dim), dtype=torch.float32, device=dev)
        if state0 is not None:
            self.slots[:, 0].copy_(torch.as_tensor(state0, dtype=torch.float32))
        self.cur = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.A = torch.as_tensor(A, dtype=torch.float32).to(dev).contiguous() if A is not None else None
        self.D = torch.as_tensor(D, dtype=torch.float32).to(dev).contiguous() if D is not None else None
        self.T_last = 0

    def verify(self, drafts: dict, y: torch.Tensor | None = None) -> torch.Tensor:
        s = self.shapes
        T = int(next(iter(drafts.values())).shape[1])
        r, keep = s.record(drafts, (s.batch, T))
        if y is None:
            y = torch.empty((s.batch, T, s.heads, s.head_dim), dtype=torch.float32, device=self.slots.device)
        B.replay_snapshot_verify(self.cfg, self.slots.data_ptr(), self.cur.data_ptr(), T,
                                 self.A.data_ptr() if self.A is not None else 0,
                                 self.D.data_ptr() if self.D is not None else 0, r, y.data_ptr(), _stream())
        self.T_last = T
        return y

    def commit(self, accepted: torch.Tensor) -> None:
        B.replay_snapshot_commit(self.cfg, self.cur.data_ptr(), accepted.data_ptr(), self.T_last, _stream())
        self.T_last = 0

    def state(self) -> torch.Tensor:
        """Current state of every sequence (a gather over the slots; test use)."""
        idx = self.cur.long()
        return self.slots[torch.arange(self.shapes.batch, device=idx.device), idx]
