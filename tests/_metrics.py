"""Error measures used by the parity tests and the bench.

Relative error of decode outputs is measured per (sequence, token): the
largest absolute difference over all of that token's head outputs, divided by
the largest magnitude among them.  A single head's output can cancel exactly
(at the first token of a Mamba-2 head y = (dt B.C + D) x, which vanishes when
dt B.C = -D), and there even the float32 stepwise recurrence is off by 1e-3
relative to that head alone; normalising by the token's output scale measures
the rounding of the computation instead of the conditioning of one head.
"""
import numpy as np


def max_rel_err(y, ref, axes=(-2, -1)):
    """Largest per-token relative error.

    y, ref: [..., heads, head_dim].  For every token (all leading axes) the
    error is ||y - ref||_inf / max(||ref||_inf, 1e-30) over its heads and
    head_dim; the maximum over tokens is returned.
    """
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.size == 0:
        return 0.0
    num = np.max(np.abs(y - ref), axis=axes)
    den = np.maximum(np.max(np.abs(ref), axis=axes), 1e-30)
    return float(np.max(num / den))
