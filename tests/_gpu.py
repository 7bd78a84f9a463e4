"""Helpers shared by the GPU parity tests (no decode arithmetic here)."""
import sys

import numpy as np


def announce(*parts):
    """Name the case before any GPU work, so a failed run still says which one."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(rec, bf16=False):
    """Device copies of a record; with bf16 the vector fields become bfloat16
    tensors (the values must already be bf16-representable: exact)."""
    import torch
    from synth import VECTOR_FIELDS
    out = {n: torch.from_numpy(np.ascontiguousarray(a)).cuda() for n, a in rec.items()}
    if bf16:
        out = {n: t.to(torch.bfloat16) if n in VECTOR_FIELDS else t for n, t in out.items()}
    return out


def host(t):
    return t.detach().cpu().numpy()


def pointers_host(layer):
    pos, ck = layer.pointers()
    return host(pos).astype(np.int64), host(ck).astype(np.int64)


def ckpt_rel_err(gpu, ref):
    """Per (sequence, head) state: max |diff| / max |ref| (state matrices)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    ax = (-2, -1)
    num = np.max(np.abs(g - r), axis=ax)
    den = np.maximum(np.max(np.abs(r), axis=ax), 1e-30)
    return float(np.max(num / den))
