"""Error measures used by the parity tests and the bench."""
import numpy as np


def max_rel_err(y, ref, axis=-1):
    """Largest per-vector relative error.

    For every output vector (the last axis: one head's output for one token of
    one sequence), ||y - ref||_inf / max(||ref||_inf, 1e-30); the maximum over
    all vectors is returned.
    """
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(y - ref), axis=axis)
    den = np.maximum(np.max(np.abs(ref), axis=axis), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0
