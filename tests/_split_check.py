"""Checks of the GPU's stored low-precision copies after a fold, and the output
bound that follows from them.  Test infrastructure (no decode arithmetic of the
library here; the oracle's codecs and replay form do the work).

After a fold the GPU's float32 fold result and the oracle's float64 one differ
by float32 rounding, so an element within that distance of a rounding boundary
(or of a stochastic-rounding threshold) may take either neighbouring code.
``check_copy`` accepts a stored code only if it is the oracle codec's encoding
of some value within delta of the oracle's fold result, with delta = rel x the
largest magnitude of the element's state row (the size of the terms the fold
sums there).  ``output_bound`` turns the accepted differences between the
GPU's and the oracle's read copy into a bound on each output: outputs are
linear in the read copy's row, with weights z (the derivative of the output
with respect to that row), so an output can move by at most sum |dQ| |z|.
"""
import numpy as np

from oracle import gdn, mamba2, quant
from oracle.session import (FMT_F16_SR, FMT_F32, FMT_F4E2M1_B16, FMT_F4E2M1_CS, FMT_F8E4M3, decode_state)

REL = 2.0 ** -15


def gpu_parts(raw, fmt, batch, shape_hpn):
    """Per-sequence stored copies (as the oracle's encode_state returns them) from
    the device bytes of one copy for the whole batch."""
    H, P, N = shape_hpn
    n = batch * H * P * N
    if fmt == FMT_F32:
        return list(raw[: 4 * n].view(np.float32).reshape(batch, H, P, N))
    if fmt == FMT_F16_SR:
        return list(raw[: 2 * n].view(np.float16).reshape(batch, H, P, N))
    if fmt == FMT_F8E4M3:
        return list(raw[:n].reshape(batch, H, P, N))
    a256 = lambda x: (x + 255) // 256 * 256
    codes = raw[: n // 2].reshape(batch, H, P, N // 2)
    off = a256(n // 2)
    scales = raw[off: off + n // 16].reshape(batch, H, P, N // 16)
    if fmt == FMT_F4E2M1_B16:
        return [(codes[b], scales[b]) for b in range(batch)]
    off2 = a256(off + n // 16)
    cols = raw[off2: off2 + batch * H * N].view(np.int8).reshape(batch, H, N)
    return [(codes[b], scales[b], cols[b]) for b in range(batch)]


def _between(lo, v, hi):
    return bool(np.all((np.minimum(lo, hi) <= v) & (v <= np.maximum(lo, hi))))


def _check_blocks(S, delta, packed, scales):
    """e2m1 blocks of 16 along the last axis: scale and codes within the window."""
    shp = S.shape[:-1] + (S.shape[-1] // 16, 16)
    blk, dblk = S.reshape(shp), np.broadcast_to(delta, S.shape).reshape(shp)
    amax, dmax = np.abs(blk).max(-1), dblk.max(-1)
    s_lo = quant.e4m3_decode(quant.e4m3_encode((np.maximum(amax - dmax, 0) / 6.0).astype(np.float32)))
    s_hi = quant.e4m3_decode(quant.e4m3_encode(((amax + dmax) / 6.0).astype(np.float32)))
    s_g = quant.e4m3_decode(scales).astype(np.float64)
    assert _between(s_lo, s_g, s_hi), "block scale outside its rounding window"
    lo = quant.e2m1_decode_values(quant.e2m1_codes_for_scale(blk - dblk, s_g)) * s_g[..., None]
    hi = quant.e2m1_decode_values(quant.e2m1_codes_for_scale(blk + dblk, s_g)) * s_g[..., None]
    lo_n, hi_n = packed & 0xF, packed >> 4
    codes = np.stack([lo_n, hi_n], axis=-1).reshape(S.shape).reshape(shp)
    got = quant.e2m1_decode_values(codes) * s_g[..., None]
    assert _between(lo, got, hi), "e2m1 code outside its rounding window"


def check_copy(parts, fmt, S_fold, seed=0, b=0, ckpt_pos=0, rel=REL):
    """Assert that one sequence's stored copy (parts, in fmt) encodes, element by
    element, a value within delta of the oracle's fold result S_fold [H, P, N];
    return the copy's decoded values (float64)."""
    S = np.asarray(S_fold, np.float64)
    delta = rel * np.abs(S).max(axis=-1, keepdims=True)
    if fmt == FMT_F32:
        assert np.all(np.abs(np.asarray(parts, np.float64) - S) <= delta), "float32 copy off the fold result"
    elif fmt == FMT_F16_SR:
        r = np.stack([quant.sr_bits(seed, b, h, ckpt_pos, S[h].size).reshape(S[h].shape) for h in range(S.shape[0])])
        lo = quant.fp16_sr((S - delta).astype(np.float32), r).astype(np.float64)
        hi = quant.fp16_sr((S + delta).astype(np.float32), r).astype(np.float64)
        assert _between(lo, np.asarray(parts, np.float64), hi), "fp16 code outside its rounding window"
    elif fmt == FMT_F8E4M3:
        lo = quant.e4m3_decode(quant.e4m3_encode((S - delta).astype(np.float32)))
        hi = quant.e4m3_decode(quant.e4m3_encode((S + delta).astype(np.float32)))
        assert _between(lo, quant.e4m3_decode(parts), hi), "e4m3 code outside its rounding window"
    elif fmt == FMT_F4E2M1_B16:
        _check_blocks(S, delta, parts[0], parts[1])
    elif fmt == FMT_F4E2M1_CS:
        packed, scales, e_g = parts
        amax = np.abs(S).max(axis=-2)                     # [H, N], over the head's rows
        dcol = delta.max(axis=-2)                         # [H, 1]
        e_lo = quant.column_exponents(np.maximum(amax - dcol, 0)[:, None, :].astype(np.float32))
        e_hi = quant.column_exponents((amax + dcol)[:, None, :].astype(np.float32))
        assert _between(e_lo.astype(int), e_g.astype(int), e_hi.astype(int)), "column exponent outside its window"
        w = np.exp2(-e_g.astype(np.float64))[:, None, :]
        _check_blocks(S * w, delta * w, packed, scales)
    else:
        raise ValueError(fmt)
    return decode_state(parts, fmt)


def query_weights(kind, recs, params=None):
    """z [H, N]: the derivative of the newest output of a window (records recs)
    with respect to any one row of the checkpoint it reads (the same for every
    row), by the oracle's replay form on an identity checkpoint with the
    record values (Mamba-2 x, GDN v) set to zero."""
    if kind == "mamba2":
        N = recs[0]["B"].shape[-1]
        H = recs[0]["x"].shape[0]
        eye = np.broadcast_to(np.eye(N), (H, N, N))
        zrec = [dict(r, x=np.zeros((H, N))) for r in recs]
        return mamba2.replay_output(eye, zrec, params["A"], np.zeros(H))
    N = recs[0]["k"].shape[-1]
    H = recs[0]["k"].shape[0]
    eye = np.broadcast_to(np.eye(N), (H, N, N))
    zrec = [dict(r, v=np.zeros((H, N))) for r in recs]
    return gdn.replay_output(eye, zrec, recs[-1]["q"])


def output_bound(dQ, z):
    """Largest move of each output element [H, P] from read-copy differences dQ [H, P, N]."""
    return np.einsum("hpn,hn->hp", np.abs(dQ), np.abs(z))


def bounded_rel_err(y, ref, scale, bound):
    """max over vectors of max(|y - ref| - bound, 0) / max(||ref||, scale)."""
    y, ref = np.asarray(y, np.float64), np.asarray(ref, np.float64)
    num = np.max(np.maximum(np.abs(y - ref) - bound, 0.0), axis=-1)
    den = np.maximum(np.maximum(np.max(np.abs(ref), axis=-1), np.asarray(scale, np.float64)), 1e-30)
    return float(np.max(num / den))
