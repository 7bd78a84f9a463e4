"""CPU checks of the post-fold checker in tests/_split_check.py: it accepts
encodings of values within its window of the fold result and rejects a code
that no such value produces (a planted mistake, on the CPU only)."""
import numpy as np
import pytest

from _split_check import REL, bounded_rel_err, check_copy, output_bound, query_weights
from oracle.session import (FMT_F16_SR, FMT_F32, FMT_F4E2M1_B16, FMT_F4E2M1_CS, FMT_F8E4M3, ReplaySession,
                            encode_state)
from synth import InputStream, LayerShape

FMTS = [FMT_F32, FMT_F16_SR, FMT_F8E4M3, FMT_F4E2M1_B16, FMT_F4E2M1_CS]


def _state(seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((2, 16, 32)) * 2.0 ** rng.integers(-3, 3, (2, 16, 1))


@pytest.mark.parametrize("fmt", FMTS)
def test_accepts_encodings_of_nearby_values(fmt):
    S = _state(1)
    rng = np.random.default_rng(2)
    delta = REL * np.abs(S).max(-1, keepdims=True)
    for trial in range(4):
        near = S + delta * rng.uniform(-0.9, 0.9, S.shape) * (trial > 0)
        parts = encode_state(near.astype(np.float32), fmt, seed=7, b=1, ckpt_pos=5)
        check_copy(parts, fmt, S, seed=7, b=1, ckpt_pos=5)


@pytest.mark.parametrize("fmt", FMTS[1:])
def test_rejects_a_wrong_code(fmt):
    S = _state(3)
    parts = encode_state(S.astype(np.float32), fmt, seed=7, b=0, ckpt_pos=4)
    if fmt == FMT_F16_SR:
        bad = parts.copy()
        bad[0, 3, 5] = np.float16(float(bad[0, 3, 5]) * 1.5 + 0.25)
    elif fmt == FMT_F8E4M3:
        bad = parts.copy()
        bad[1, 2, 7] ^= 0x10                              # an exponent bit: far from any rounding window
    else:
        packed = parts[0].copy()
        packed[0, 0, 3] ^= 0x06                           # a magnitude two codes away
        bad = (packed,) + tuple(parts[1:])
    with pytest.raises(AssertionError):
        check_copy(bad, fmt, S, seed=7, b=0, ckpt_pos=4)


def test_rejects_a_wrong_block_scale():
    S = _state(4)
    packed, scales = encode_state(S.astype(np.float32), FMT_F4E2M1_B16)
    scales = scales.copy()
    scales[1, 4, 1] += 1
    with pytest.raises(AssertionError):
        check_copy((packed, scales), FMT_F4E2M1_B16, S)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_output_bound_covers_a_read_copy_change(kind):
    """The bound from query_weights is exact for a change of one read-copy row
    (outputs are linear in it) and covers any change of the copy."""
    shape = LayerShape(kind, 1, 2, 32, 32, 1 if kind == "mamba2" else 2, 4)
    ins = InputStream(shape, 6)
    S0 = ins.initial_state(zeros=False, scale=0.3)[0]
    recs = []
    for _ in range(3):
        r = ins.record()
        recs.append({n: a[0] for n, a in r.items()})
    out = lambda S: ReplaySession(kind, S[None], 4, ins.params).k.output(S, recs)
    z = query_weights(kind, recs, ins.params)
    rng = np.random.default_rng(8)
    S0 = S0.astype(np.float64)
    dQ = np.zeros(S0.shape)
    dQ[1, 5, :] = rng.standard_normal(32) * 1e-3
    dy = out(S0 + dQ) - out(S0)
    np.testing.assert_allclose(dy[1, 5], dQ[1, 5] @ z[1], rtol=1e-9, atol=1e-15)
    dQ = rng.standard_normal(S0.shape) * 1e-3
    dy = out(S0 + dQ) - out(S0)
    assert np.all(np.abs(dy) <= output_bound(dQ, z) * (1 + 1e-9) + 1e-15)
    assert bounded_rel_err(out(S0 + dQ), out(S0), np.zeros(2), output_bound(dQ, z)) <= 1e-12
