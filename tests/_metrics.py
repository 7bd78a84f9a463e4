"""Error measure used by the parity tests and the bench.

The relative error of decode outputs is measured per output vector: one head
of one sequence at one token (b, h, t), the head_dim values of that head.
Its denominator is the larger of the reference vector's largest magnitude and
the size of the terms the output sums (``scale``, from the oracle sessions:
Mamba-2 max_p (|S| |C|)_p + |D| max |x|; Gated DeltaNet max_v (|S| |q|)_v, S
the state the output reads).  A head's output can cancel (at the first token
of a Mamba-2 head y = (dt B.C + D) x, which vanishes when dt B.C = -D); there
any float32 evaluation is off relative to the small result, and the second
term measures the rounding of the sum instead of the conditioning of the
head.  No head borrows the scale of another.
"""
import numpy as np


def max_rel_err(y, ref, scale=None):
    """Largest per-vector relative error.

    y, ref: [..., head_dim], one vector per leading index; scale: [...] (the
    leading axes) or None.  For every vector the error is
    ||y - ref||_inf / max(||ref||_inf, scale, 1e-30); the maximum is returned.
    """
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.size == 0:
        return 0.0
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    if scale is not None:
        den = np.maximum(den, np.asarray(scale, np.float64))
    return float(np.max(num / np.maximum(den, 1e-30)))
