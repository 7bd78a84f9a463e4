"""Pins for the split-precision codecs and the Philox generator.

Against published values (Philox known-answer vectors), a library cast
(torch.float8_e4m3fn on inputs already inside +-448), exhaustive enumeration
of every code, hand-placed rounding ties, and statistical properties of the
stochastic rounding.
"""
import numpy as np
import pytest

from oracle import quant


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library (Philox-4x32, 10 rounds).
    cases = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in cases:
        got = quant.philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
        assert [int(v) for v in got] == want


def test_e4m3_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = quant.e4m3_decode(codes)
    ok = ~np.isnan(vals) & (codes != 0x80)            # NaN codes and -0 are never produced
    assert np.array_equal(quant.e4m3_encode(vals[ok]), codes[ok])
    assert quant.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert quant.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9
    assert quant.e4m3_decode(np.array([0x08], np.uint8))[0] == 2.0 ** -6


def test_e4m3_ties_to_even_and_saturation():
    pos = np.arange(0x7F, dtype=np.uint8)              # 0 .. 0x7E
    v = quant.e4m3_decode(pos).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)   # exact in float32
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)
    got = quant.e4m3_encode(mids)
    want = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, want)
    assert np.array_equal(quant.e4m3_encode(np.array([448.0, 460.0, 1e9, np.inf], np.float32)),
                          np.full(4, 0x7E, np.uint8))
    assert quant.e4m3_encode(np.array([-1e9], np.float32))[0] == 0xFE
    assert quant.e4m3_encode(np.array([2.0 ** -11, -2.0 ** -11], np.float32)).tolist() == [0, 0]


def test_e4m3_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000),
                        rng.uniform(-2.0 ** -6, 2.0 ** -6, 50000)]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)                      # torch's cast does not saturate; the codec does
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where(ref == 0x80, 0, ref)                # the codec never writes -0; torch keeps the sign
    assert np.array_equal(quant.e4m3_encode(x), ref)


def test_e2m1_codes_and_ties():
    codes = np.arange(16, dtype=np.uint8)
    vals = quant.e2m1_decode_values(codes)
    ok = codes != 8                                     # -0 is never produced
    assert np.array_equal(quant.e2m1_encode_values(vals[ok]), codes[ok])
    # midpoints between neighbouring grid values round to the even code
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert quant.e2m1_encode_values(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert quant.e2m1_encode_values(-ties).tolist() == [0, 10, 10, 12, 12, 14, 14]
    assert quant.e2m1_encode_values(np.array([7.0, -100.0], np.float32)).tolist() == [7, 15]


def test_e2m1_block_format():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((5, 64)) * np.array([1e-3, 1.0, 30.0, 1e3, 0.0])[:, None]).astype(np.float32)
    packed, scales = quant.e2m1_block_encode(x)
    assert packed.shape == (5, 32) and scales.shape == (5, 4)
    xd = quant.e2m1_block_decode(packed, scales)
    assert np.all(xd[4] == 0) and np.all(scales[4] == 0)
    # every element lies on its block's grid, and the error is at most half a grid step
    # (the largest step is 2 s at |y| in [4, 6]), or the clamp at 6 s
    s = quant.e4m3_decode(scales).astype(np.float64)
    err = np.abs(xd.astype(np.float64) - x).reshape(5, 4, 16)
    clamp = np.maximum(np.abs(x).reshape(5, 4, 16) - 6 * s[..., None], 0)
    assert np.all(err <= s[..., None] + clamp + 1e-12)
    # the low nibble holds the even element
    lo = quant.e2m1_decode_values(packed[0, :1] & 0xF)[0] * s[0, 0]
    assert lo == xd[0, 0]


def test_fp16_sr_fixed_points_and_saturation():
    rng = np.random.default_rng(2)
    f16 = rng.standard_normal(4000).astype(np.float16)
    f16 = np.concatenate([f16, np.array([2.0 ** -24, -2.0 ** -20, 65504, -65504, 0.0], np.float16)])
    x = f16.astype(np.float32)
    for r in (0, 1, 2 ** 23, 2 ** 24 - 1):
        assert np.array_equal(quant.fp16_sr(x, np.full(x.shape, r)), f16)
    big = np.array([7e4, -1e9, np.inf], np.float32)
    assert quant.fp16_sr(big, np.array([2 ** 24 - 1] * 3)).tolist() == [65504.0, -65504.0, 65504.0]


def test_fp16_sr_zero_bits_truncate_and_mean_is_unbiased():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(64) * 10.0 ** rng.integers(-6, 4, 64)).astype(np.float32)
    rtz = quant.fp16_sr(x, np.zeros(64, np.int64)).astype(np.float64)
    rn = x.astype(np.float16).astype(np.float64)
    # r = 0 is round toward zero: never above |x|, and within one fp16 step of round-to-nearest
    assert np.all(np.abs(rtz) <= np.abs(x.astype(np.float64)))
    assert np.all((rtz == rn) | (np.abs(rn) > np.abs(x.astype(np.float64))))
    # E[SR(x)] = x: average over 2^16 random draws, within 5 standard errors of one fp16 step
    for xi in x[:16]:
        r = rng.integers(0, 2 ** 24, 1 << 16)
        vals = quant.fp16_sr(np.full(r.shape, xi, np.float32), r).astype(np.float64)
        step = np.spacing(np.float16(abs(xi))).astype(np.float64)
        assert abs(vals.mean() - float(xi)) <= 5 * step / 2 / np.sqrt(len(r)) + 1e-30


# ---- two-axis e2m1 (block scales along the state axis, a power-of-two scale per column) ----
def test_column_exponents_rule():
    """e = floor(log2 amax) - 5 (so amax / 2^e is in [32, 64)), clamped at -126; zero columns -126."""
    S = np.zeros((3, 6), np.float32)
    S[1] = [1.0, -0.75, 64.0, 2.0 ** -130, 0.0, 3e38]
    S[2, 0] = -0.5                                   # smaller than the column maximum: no effect
    e = quant.column_exponents(S)
    assert e.dtype == np.int8
    assert e.tolist() == [-5, -6, 1, -126, -126, 122]
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((4, 8, 32)) * 2.0 ** rng.integers(-30, 30, (4, 1, 32))).astype(np.float32)
    e = quant.column_exponents(X).astype(np.float64)
    ratio = np.max(np.abs(X), axis=-2) / 2.0 ** e
    assert np.all((ratio >= 32) & (ratio < 64))


def test_two_axis_column_scaling_is_equivariant():
    """Scaling a column by 2^k moves only its exponent: codes, block scales and the rest stay."""
    rng = np.random.default_rng(8)
    S = rng.standard_normal((2, 16, 32)).astype(np.float32)
    p0, s0, e0 = quant.e2m1_cs_encode(S)
    T = S.copy()
    T[:, :, 5] *= 2.0 ** 9
    T[:, :, 20] *= 2.0 ** -7
    p1, s1, e1 = quant.e2m1_cs_encode(T)
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)
    de = e1.astype(int) - e0.astype(int)
    assert np.all(de[:, 5] == 9) and np.all(de[:, 20] == -7) and np.count_nonzero(de) == 4
    D0, D1 = quant.e2m1_cs_decode(p0, s0, e0), quant.e2m1_cs_decode(p1, s1, e1)
    assert np.array_equal(D1[:, :, 5], D0[:, :, 5] * 2.0 ** 9)
    assert np.array_equal(D1[:, :, 20], D0[:, :, 20] * 2.0 ** -7)
    # the block format alone is not equivariant: a 2^9 column takes over its blocks
    b0 = quant.e2m1_block_decode(*quant.e2m1_block_encode(S))
    b1 = quant.e2m1_block_decode(*quant.e2m1_block_encode(T))
    assert not np.array_equal(b1[:, :, 4], b0[:, :, 4])


def test_two_axis_grid_and_error_bound():
    """Each decoded element / 2^e lies on its block's e2m1 grid, within half the largest step."""
    rng = np.random.default_rng(9)
    S = (rng.standard_normal((3, 16, 64)) * np.exp(2 * rng.standard_normal((3, 1, 64)))).astype(np.float32)
    S[0, :, 3] = 0.0                                 # an all-zero column
    p, sc, e = quant.e2m1_cs_encode(S)
    D = quant.e2m1_cs_decode(p, sc, e)
    assert np.all(D[0, :, 3] == 0)
    y = D / 2.0 ** e.astype(np.float64)[:, None, :]
    s = quant.e4m3_decode(sc).astype(np.float64)                       # [3, 16, 4]
    blk = y.reshape(3, 16, 4, 16) / np.where(s > 0, s, 1.0)[..., None]
    assert np.all(np.isin(np.abs(blk), quant.E2M1_GRID.astype(np.float64)))
    x = (S.astype(np.float64) / 2.0 ** e.astype(np.float64)[:, None, :]).reshape(3, 16, 4, 16)
    clamp = np.maximum(np.abs(x) - 6 * s[..., None], 0)
    assert np.all(np.abs(y.reshape(3, 16, 4, 16) - x) <= s[..., None] + clamp + 1e-12)
    # a block of equal magnitudes on one grid point is reproduced exactly
    Z = np.full((1, 16, 16), 3.0, np.float32) * np.array([1, -1] * 8, np.float32)
    assert np.array_equal(quant.e2m1_cs_decode(*quant.e2m1_cs_encode(Z)), Z.astype(np.float64))
