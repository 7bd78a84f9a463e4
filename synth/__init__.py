"""Seeded synthetic inputs for the Mamba-2 and Gated DeltaNet decode layers.

This module draws random numbers and gives them shapes.  It holds none of the
decode arithmetic: the CPU oracle and the HIP library both receive the float32
arrays produced here, so the two sides always see identical bytes.

Draw order is fixed so that a (workload, seed) pair names one input stream:
the layer parameters first (Mamba-2: ``A`` then ``D``), then for every decode
step one array per record field, in record order.  Speculative drafts are
drawn as ``[batch, T, ...]`` arrays, field by field, followed by the accepted
lengths.  Every draw is made in float64 by ``numpy.random.Generator(PCG64(seed))``
and cast to float32.

Value distributions (the workloads the pages measure are real model layers;
these synthetic stand-ins use the same shapes and plausible value ranges):

* Mamba-2: x, B, C ~ N(0, 1); dt = softplus(N(0, 1) - 2); A = -exp(U(0, ln 16));
  D ~ N(0, 1).
* Gated DeltaNet: q, k ~ N(0, 1), each then scaled to unit L2 norm per head;
  v ~ N(0, 1); beta = sigmoid(N(0, 1)); alpha = exp(-0.1 * softplus(N(0, 1))).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MAMBA2 = "mamba2"
GDN = "gdn"


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


VECTOR_FIELDS = ("x", "B", "C", "q", "k", "v")


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), kept as float32
    (finite inputs): records that a bf16 tensor holds exactly."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(np.shape(a))


@dataclass(frozen=True)
class LayerShape:
    """Shape of one decode layer.

    kind: ``"mamba2"`` or ``"gdn"``.
    head_dim: Mamba-2 P, GDN d_v.  state_dim: Mamba-2 N, GDN d_k.
    groups: Mamba-2 B/C groups (heads are split into contiguous blocks of
    heads // groups); GDN uses groups == heads.
    """

    kind: str
    batch: int
    heads: int
    head_dim: int
    state_dim: int
    groups: int
    window: int

    def state_elems_per_seq(self) -> int:
        return self.heads * self.head_dim * self.state_dim


# Named workloads: the shapes of the layers the pages measure, at the sizes
# used for parity and timing.
WORKLOADS = {
    # Small Mamba-2 layer for exhaustive parity: every output of every step.
    "mamba2_b2_h4_p16_n16_l4": LayerShape(MAMBA2, 2, 4, 16, 16, 1, 4),
    # Mamba-2 layer whose FP32 state is 4 MiB per sequence, at batch 256.
    "mamba2_b256_h128_p64_n128_g8_l16": LayerShape(MAMBA2, 256, 128, 64, 128, 8, 16),
    # Gated DeltaNet layer, 2 MiB FP32 state per sequence, batch 256.
    "gdn_b256_h32_d128_l16": LayerShape(GDN, 256, 32, 128, 128, 32, 16),
    # Speculative verify: the 4 MiB Mamba-2 layer at batch 512.
    "mamba2_b512_h128_p64_n128_g8_l16": LayerShape(MAMBA2, 512, 128, 64, 128, 8, 16),
    # Split-precision state: the Gated DeltaNet layer at batch 64.
    "gdn_b64_h32_d128_l16": LayerShape(GDN, 64, 32, 128, 128, 32, 16),
}


def field_names(kind: str) -> tuple[str, ...]:
    """Record fields in draw (and ABI) order."""
    return ("x", "B", "C", "dt") if kind == MAMBA2 else ("q", "k", "v", "alpha", "beta")


class InputStream:
    """Seeded stream of layer parameters, decode records and speculative drafts.

    ``lead`` axes: a record has shape ``[batch, ...]`` per field; drafts have
    ``[batch, T, ...]``.
    """

    def __init__(self, shape: LayerShape, seed: int, bf16_vectors: bool = False):
        """bf16_vectors: the vector fields (x, B, C / q, k, v) are rounded to bf16
        values after drawing (the same draws, so the stream stays aligned)."""
        self.shape = shape
        self.bf16_vectors = bf16_vectors
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.params = self._draw_params()

    # -- parameters ---------------------------------------------------------
    def _draw_params(self) -> dict[str, np.ndarray]:
        s = self.shape
        if s.kind != MAMBA2:
            return {}
        A = -np.exp(self.rng.uniform(0.0, np.log(16.0), size=s.heads))
        D = self.rng.standard_normal(s.heads)
        return {"A": A.astype(np.float32), "D": D.astype(np.float32)}

    # -- records ------------------------------------------------------------
    def _draw(self, lead: tuple[int, ...]) -> dict[str, np.ndarray]:
        s, r = self.shape, self.rng
        if s.kind == MAMBA2:
            x = r.standard_normal(lead + (s.heads, s.head_dim))
            B = r.standard_normal(lead + (s.groups, s.state_dim))
            C = r.standard_normal(lead + (s.groups, s.state_dim))
            dt = _softplus(r.standard_normal(lead + (s.heads,)) - 2.0)
            out = {"x": x, "B": B, "C": C, "dt": dt}
        else:
            q = r.standard_normal(lead + (s.heads, s.state_dim))
            k = r.standard_normal(lead + (s.heads, s.state_dim))
            q /= np.linalg.norm(q, axis=-1, keepdims=True)
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
            v = r.standard_normal(lead + (s.heads, s.head_dim))
            alpha = np.exp(-0.1 * _softplus(r.standard_normal(lead + (s.heads,))))
            beta = _sigmoid(r.standard_normal(lead + (s.heads,)))
            out = {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}
        out = {n: np.ascontiguousarray(a.astype(np.float32)) for n, a in out.items()}
        if self.bf16_vectors:
            out = {n: round_to_bf16(a) if n in VECTOR_FIELDS else a for n, a in out.items()}
        return out

    def record(self) -> dict[str, np.ndarray]:
        """One decode token for every sequence: fields shaped [batch, ...]."""
        return self._draw((self.shape.batch,))

    def drafts(self, T: int) -> dict[str, np.ndarray]:
        """T draft tokens per sequence: fields shaped [batch, T, ...]."""
        return self._draw((self.shape.batch, T))

    def accepted(self, T: int) -> np.ndarray:
        """Accepted draft count per sequence, uniform over 0..T, int32 [batch]."""
        return self.rng.integers(0, T + 1, size=self.shape.batch).astype(np.int32)

    def initial_state(self, zeros: bool = True, scale: float = 1.0) -> np.ndarray:
        """Initial checkpoint [batch, heads, head_dim, state_dim] float32.

        Zeros by default; ``zeros=False`` draws N(0, scale^2) entries, used by
        tests that need a non-trivial checkpoint.
        """
        s = self.shape
        shp = (s.batch, s.heads, s.head_dim, s.state_dim)
        if zeros:
            return np.zeros(shp, np.float32)
        return (scale * self.rng.standard_normal(shp)).astype(np.float32)


def take_batch(rec: dict[str, np.ndarray], idx) -> dict[str, np.ndarray]:
    """Rows ``idx`` of every field (the sequences an oracle check samples)."""
    return {n: np.ascontiguousarray(a[idx]) for n, a in rec.items()}


class DeviceInputStream:
    """Seeded decode records generated on the GPU with torch, for long runs
    (tens of thousands of steps) where host-side arrays would be too large.

    Same distributions as InputStream; the random numbers come from a seeded
    torch generator on the device, so the stream is reproducible but is not
    the same stream as InputStream's.  Only Gated DeltaNet layers.
    """

    def __init__(self, shape: LayerShape, seed: int, device="cuda", key_spread: float = 0.0,
                 bf16_vectors: bool = False):
        """key_spread > 0 gives every (head, key dimension) of q and of k a fixed
        magnitude weight exp(key_spread N(0, 1)) (drawn once, before the first
        record) applied before the L2 normalisation: key dimensions of uneven
        size, hence state columns of uneven magnitude."""
        import torch
        if shape.kind != GDN:
            raise ValueError("DeviceInputStream generates Gated DeltaNet records")
        self.torch = torch
        self.shape = shape
        self.gen = torch.Generator(device=device)
        self.gen.manual_seed(seed)
        self.device = device
        self.bf16_vectors = bf16_vectors  # q, k, v returned as bfloat16 tensors
        self.wq = self.wk = None
        if key_spread > 0:
            w = lambda: torch.exp(key_spread * torch.randn(shape.heads, shape.state_dim, generator=self.gen,  # noqa: E731
                                                           device=device, dtype=torch.float32))
            self.wq, self.wk = w(), w()

    def record(self):
        t, s = self.torch, self.shape
        lead = (s.batch, s.heads)
        n = lambda *shp: t.randn(*shp, generator=self.gen, device=self.device, dtype=t.float32)  # noqa: E731
        q = n(*lead, s.state_dim)
        k = n(*lead, s.state_dim)
        if self.wq is not None:
            q, k = q * self.wq, k * self.wk
        q = q / t.linalg.vector_norm(q, dim=-1, keepdim=True)
        k = k / t.linalg.vector_norm(k, dim=-1, keepdim=True)
        v = n(*lead, s.head_dim)
        alpha = t.exp(-0.1 * t.nn.functional.softplus(n(*lead)))
        beta = t.sigmoid(n(*lead))
        if self.bf16_vectors:
            q, k, v = (x.to(t.bfloat16) for x in (q, k, v))
        return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(), "alpha": alpha.contiguous(),
                "beta": beta.contiguous()}
