"""OCP 8-bit floating point E4M3 for the expert and LM-head weights (oracle side).

The pages give the deployed model's weights in FP8 (chooseai.io speed
paragraph: the vLLM FP8 figures; bohuyeshan.top 一: the quantised model runs
in 18 GB), without the format's details.  Reading: the OCP FP8 "E4M3"
encoding (Open Compute Project, "OCP 8-bit Floating Point Specification
(OFP8)", rev. 1.0): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 holds subnormals m * 2^-9; there are no infinities;
S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
Conversion rounds to nearest, ties to even, and saturates to +-448 (the
specification's saturating mode).

Scaling (a reading; the pages name none): one fp32 scale per output channel
of each expert matrix (a row of the [out, in] layout) and of the LM head (a
row of E, one vocabulary id),
    scale = fl32(fl64(max |w_row|) / 448)     (1.0 for an all-zero row),
    q     = E4M3(fl32(w / scale))             (an fp32 division, then the conversion),
and the weight the model uses is q * scale (exact in fp64).
"""
from __future__ import annotations

import numpy as np

MAX_NORMAL = 448.0
EXP_BIAS = 7


def decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> values (fp64).  NaN codes (0x7F, 0xFF) decode to NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - EXP_BIAS))
    val = np.where((e == 0xF) & (m == 7), np.nan, val)
    return sign * val


def encode(x) -> np.ndarray:
    """Values -> E4M3 codes, round to nearest even, saturating at +-448."""
    x = np.asarray(x, np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, np.int64)
    # subnormal range: a < 2^-6 -> m = rne(a / 2^-9) in 0..8 (8 is the smallest normal, code 0x08)
    sub = a < 2.0 ** -6
    ms = np.rint(a * 2.0 ** 9).astype(np.int64)           # exact scaling; rint rounds half to even
    out = np.where(sub, ms, out)                          # ms == 8 is exactly code 0x08
    # normal range: a = (1 + f) 2^e, e in -6..8; mantissa rne((a / 2^e - 1) * 8)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    frac = np.where(sub, 1.0, a / np.exp2(e.astype(np.float64)))
    # log2 of a value just below a power of two can come out at the power: fix the exponent
    lo = frac < 1.0
    e = np.where(lo, e - 1, e)
    frac = np.where(lo, frac * 2.0, frac)
    mm = np.rint((frac - 1.0) * 8.0).astype(np.int64)
    carry = mm == 8
    e = np.where(carry, e + 1, e)
    mm = np.where(carry, 0, mm)
    norm = ((e + EXP_BIAS) << 3) | mm
    over = (a > MAX_NORMAL) | (e > 8)
    norm = np.where(over, 0x7E, norm)                     # saturate to 448
    out = np.where(sub, out, norm)
    return (sign | out).astype(np.uint8)


def row_scales(w) -> np.ndarray:
    """Per-row scales of a [..., rows, cols] matrix: fl32(fl64(max |w_row|) / 448), 1 for zero rows."""
    w = np.asarray(w, np.float32)
    amax = np.abs(w).max(axis=-1).astype(np.float64)
    s = (amax / MAX_NORMAL).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_rows(w):
    """[..., rows, cols] weights (fp32 values) -> (codes uint8, scales fp32 [..., rows])."""
    w = np.asarray(w, np.float32)
    s = row_scales(w)
    v = w / s[..., None]                                   # fp32 division
    return encode(v.astype(np.float64)), s


def dequantize_rows(codes, scales) -> np.ndarray:
    """codes [..., rows, cols], scales [..., rows] -> fp64 weights q * scale."""
    return decode(codes) * np.asarray(scales, np.float64)[..., None]
