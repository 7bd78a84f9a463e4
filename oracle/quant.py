"""Storage codecs of the split-precision state.  Test infrastructure only.

The pages separate the precision of the recurrence checkpoint from that of
the copy read for outputs: a low-precision read copy whose rounding never
re-enters the recurrence, against a shared low-precision checkpoint whose
rounding is written back at every fold and accumulates [P1, Interpretation 4;
P1, Perspective 2; P3, Interpretation 3].  They name NVFP4 reads and FP16
(with stochastic rounding) or FP8 recurrences without defining the codecs;
the definitions below are the readings taken (plain, and the same on both the
CPU and the GPU side, so that every rounding decision is bit-identical):

* e4m3 (OCP FP8 e4m3fn): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
  round to nearest, ties to even; saturates at +-448; no scale.
* e2m1 block format: 4-bit e2m1 values {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a
  sign bit, one e4m3 scale per block of 16 consecutive elements along the
  state's contiguous dimension: s = e4m3(amax / 6) (amax / 6 a correctly
  rounded float32 division); a block with s == 0 is all zero; each element is
  x / s clamped to +-6 and rounded to the nearest grid value, ties to the even
  code, decided exactly by comparing |x| with the midpoints t s (t in 0.25,
  0.75, 1.25, 1.75, 2.5, 3.5, 5; every t s is exact in float32); a zero
  magnitude carries no sign.  Two codes per byte, the even element in the low
  nibble.
* two-axis e2m1 (a reading of the pages' suggestion of separate scales along
  the state and channel dimensions for the read copy [P1, Perspective 2]):
  the block scales above run along the state axis inside one
  channel row; in addition every state column n of a head has a power-of-two
  scale 2^e[n] (one signed byte), e = max(floor(log2 amax_n) - 5, -126) from
  the column's largest magnitude over the head's channels (-126 for a zero
  column).  The element codes and block scales are the block format of
  S[p, n] / 2^e[n] (an exact division unless the quotient is subnormal), and
  the decoded value is e2m1 x block scale x 2^e[n].
* fp16 with stochastic rounding: SR(x, r) = RTZ_fp16(x + sign(x) (r / 2^24)
  ulp16(|x|)) for a 24-bit random integer r, saturating at +-65504, where
  ulp16 is the binary16 spacing at |x| (2^-24 below 2^-14).

All functions take and return NumPy arrays; float inputs are float32.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
FP16_MAX = 65504.0


# ---- e4m3 ------------------------------------------------------------------------
def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return (sign * mag).astype(np.float32)


def e4m3_encode(x) -> np.ndarray:
    """float32 -> e4m3 code, round to nearest even, saturating."""
    x = np.asarray(x, np.float32)
    out = np.zeros(x.shape, np.uint8)
    a = np.abs(x).astype(np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    e = (bits >> 23) - 127
    mant = bits & 0x7FFFFF
    # normal e4m3 range: |x| >= 2^-6; 3 of the 23 mantissa bits survive
    r = mant >> 20
    rem = mant & ((1 << 20) - 1)
    up = (rem > (1 << 19)) | ((rem == (1 << 19)) & ((r & 1) == 1))
    r = r + up
    e_n = np.where(r == 8, e + 1, e)
    r = np.where(r == 8, 0, r)
    code_n = ((e_n + 7) << 3) | r
    code_n = np.minimum(code_n, 0x7E)
    # subnormal e4m3 range: steps of 2^-9, round half to even
    q = np.rint(np.minimum(a, 1.0).astype(np.float64) * 512.0).astype(np.int64)  # exact: a * 2^9
    code_s = np.minimum(q, 8)
    code = np.where(a >= 2.0 ** -6, code_n, code_s)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    sign = np.where((x < 0) & (code != 0), 0x80, 0)
    out[...] = (code | sign).astype(np.uint8)
    return out


# ---- e2m1 with an e4m3 scale per block of 16 ------------------------------------------
def e2m1_encode_values(y) -> np.ndarray:
    """Already-scaled float32 values -> 4-bit codes (sign in bit 3)."""
    y = np.asarray(y, np.float32)
    a = np.minimum(np.abs(y), np.float32(6.0))
    mag = np.select([a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
                    [0, 1, 2, 3, 4, 5, 6], default=7).astype(np.uint8)
    sign = np.where((y < 0) & (mag != 0), 8, 0).astype(np.uint8)
    return mag | sign


def e2m1_decode_values(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    v = E2M1_GRID[c & 7]
    return np.where(c & 8, -v, v).astype(np.float32)


def e2m1_block_encode(x):
    """x [..., n] float32 (n a multiple of 16) -> (packed codes [..., n/2] uint8, scales [..., n/16] uint8)."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    if n % 16:
        raise ValueError("last axis must be a multiple of 16")
    blk = x.reshape(x.shape[:-1] + (n // 16, 16))
    amax = np.max(np.abs(blk), axis=-1)
    scode = e4m3_encode((amax / np.float32(6.0)).astype(np.float32))
    codes = e2m1_codes_for_scale(blk, e4m3_decode(scode)).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scode


def e2m1_codes_for_scale(blk, s) -> np.ndarray:
    """4-bit codes of the elements blk [..., 16] under the block scales s [...]
    (decoded e4m3 values): |x| against the midpoints t s of the grid, ties to
    the even code, clamped at 6 s; all zero where s == 0."""
    s = np.asarray(s, np.float64)[..., None]
    blk = np.asarray(blk, np.float64)
    a = np.abs(blk)
    mag = np.select([a <= 0.25 * s, a < 0.75 * s, a <= 1.25 * s, a < 1.75 * s, a <= 2.5 * s, a < 3.5 * s,
                     a <= 5.0 * s], [0, 1, 2, 3, 4, 5, 6], default=7).astype(np.uint8)
    mag = np.where(s > 0, mag, 0).astype(np.uint8)
    sign = np.where((blk < 0) & (mag != 0), 8, 0).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def e2m1_block_decode(packed, scales) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    vals = e2m1_decode_values(codes)
    s = e4m3_decode(scales)
    n = vals.shape[-1]
    return (vals.reshape(vals.shape[:-1] + (n // 16, 16)) * s[..., None]).reshape(vals.shape).astype(np.float32)


# ---- e2m1 with block scales along the state axis and a scale per state column ----------
def column_exponents(S) -> np.ndarray:
    """S [..., P, N] float32 -> int8 e[..., N]: column n of each head takes the scale 2^e[n],
    e = max(floor(log2 amax_n) - 5, -126) with amax_n = max_p |S[p, n]| (e = -126 for an
    all-zero column), so that the column's largest magnitude divided by 2^e lies in [32, 64)."""
    S = np.asarray(S, np.float32)
    amax = np.max(np.abs(S), axis=-2).astype(np.float64)
    _, ex = np.frexp(amax)                       # amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
    e = np.where(amax > 0, ex - 1 - 5, -126)
    return np.maximum(e, -126).astype(np.int8)


def e2m1_cs_encode(S):
    """S [..., P, N] float32 -> (packed codes [..., P, N/2], block scales [..., P, N/16],
    column exponents [..., N] int8): the e2m1 block format of S[p, n] / 2^e[n]."""
    S = np.asarray(S, np.float32)
    e = column_exponents(S)
    y = (S.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None, :]).astype(np.float32)
    packed, scales = e2m1_block_encode(y)
    return packed, scales, e


def e2m1_cs_decode(packed, scales, e) -> np.ndarray:
    """Float64 value of each element: e2m1 value x block scale x 2^e[column] (exact)."""
    y = e2m1_block_decode(packed, scales).astype(np.float64)
    return y * np.exp2(np.asarray(e, np.float64))[..., None, :]


# ---- fp16 with stochastic rounding ------------------------------------------------------
def fp16_sr(x, r24) -> np.ndarray:
    """float32 x, 24-bit integers r24 -> float16 (stochastically rounded, saturating)."""
    x = np.asarray(x, np.float32)
    r = np.asarray(r24, np.int64) & 0xFFFFFF
    a = np.abs(x)
    bits = a.view(np.uint32).astype(np.int64)
    # fp16 normal range: add the top 13 random bits below the fp16 mantissa and truncate
    t = (bits + (r >> 11)) & ~np.int64(0x1FFF)
    normal = t.astype(np.uint32).view(np.float32).astype(np.float64)
    # fp16 subnormal range: units of 2^-24
    v = np.minimum(a, 1.0).astype(np.float64) * 2.0 ** 24     # exact (only a < 2^-14 is used)
    n = np.floor(v)
    f = (v - n).astype(np.float32)
    thr = ((2 ** 24 - r).astype(np.float64) * 2.0 ** -24).astype(np.float32)
    sub = (n + (f >= thr)) * 2.0 ** -24
    mag = np.where(a >= 2.0 ** -14, normal, sub)
    mag = np.minimum(mag, FP16_MAX)
    return (np.sign(x) * mag).astype(np.float16)


# ---- Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
# 1, 2, 3", SC'11) ------------------------------------------------------------------------
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key) -> np.ndarray:
    """ctr [..., 4] uint32, key [..., 2] uint32 -> [..., 4] uint32."""
    c = np.asarray(ctr, np.uint64) & 0xFFFFFFFF
    k = np.asarray(key, np.uint64) & 0xFFFFFFFF
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    M = np.uint64(0xFFFFFFFF)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & M
            k1 = (k1 + np.uint64(PHILOX_W1)) & M
        p0 = np.uint64(PHILOX_M0) * c0
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & M
        hi1, lo1 = p1 >> np.uint64(32), p1 & M
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def sr_bits(seed: int, b: int, h: int, ckpt_pos: int, n_elems: int) -> np.ndarray:
    """24-bit random integers for the n_elems elements (row-major) of one head's state,
    written by the fold that sets ckpt_pos of sequence b: counter (e // 4, h, b, ckpt_pos),
    key (seed low, seed high), element e takes word e % 4, top 24 bits."""
    e4 = np.arange((n_elems + 3) // 4, dtype=np.uint64)
    ctr = np.stack([e4, np.full_like(e4, h), np.full_like(e4, b), np.full_like(e4, ckpt_pos)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint64)
    words = philox4x32_10(ctr, key).reshape(-1)[:n_elems]
    return (words >> np.uint32(8)).astype(np.int64)
