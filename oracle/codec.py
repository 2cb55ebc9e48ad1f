"""FP8 E4M3 codec and bf16 rounding (oracle; test infrastructure only).

The pages say only "FP8" ([KANANA-FP8], [DSV3-FP8]).  Reading taken here:
the OCP 8-bit E4M3 format in its "FN" flavour (no infinities), i.e.
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
holds subnormals m * 2^-9; the single NaN pattern per sign is S.1111.111, so
the largest finite magnitude is 1.75 * 2^8 = 448.  Encoding rounds to the
nearest representable value with ties to the even mantissa and keeps the sign
(so -0 and negative values that round to zero give 0x80).
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each E4M3FN code as float64 (NaN for 0x7F / 0xFF).

    Field layout from the format definition: s = bit 7, e = bits 6..3,
    m = bits 2..0; e == 0 -> (-1)^s * m * 2^-9; otherwise
    (-1)^s * (1 + m/8) * 2^(e-7); e == 15 and m == 7 -> NaN.
    """
    c = np.asarray(codes).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_values():
    """The 127 non-negative finite magnitudes, indexed by code 0x00..0x7E."""
    return e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v):
    """Round finite values with |v| <= 448 to E4M3FN codes (RNE, sign kept).

    Plain algorithm: the spacing of representable values in the binade
    [2^e, 2^(e+1)) is 2^(e-3) for e >= -6 and 2^-9 below (subnormals);
    divide by that spacing (exact: a power of two), round half to even,
    multiply back, then read the fields off the rounded value.  A value that
    rounds up to the next power of two is still exactly representable.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values with |v| <= 448")
    neg = np.signbit(v)
    a = np.abs(v)
    _, ex = np.frexp(a)                    # a = f * 2^ex, f in [0.5, 1)
    e_unb = np.maximum(ex - 1, -6)          # binade exponent, subnormal floor
    spacing = np.exp2(e_unb.astype(np.float64) - 3.0)
    q = np.rint(a / spacing) * spacing      # np.rint rounds half to even
    # fields of the rounded magnitude q (0 <= q <= 448)
    _, qe = np.frexp(q)
    qe = qe - 1
    is_normal = q >= 2.0 ** -6
    e_field = np.where(is_normal, qe + 7, 0)
    m_normal = (q / np.exp2(qe.astype(np.float64)) - 1.0) * 8.0
    m_sub = q / 2.0 ** -9
    m_field = np.where(is_normal, m_normal, m_sub)
    code = (e_field.astype(np.int64) << 3) | np.rint(m_field).astype(np.int64)
    code = np.where(q == 0, 0, code)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def e4m3_encode_bruteforce(v):
    """Second encoder for cross-checking: nearest of the 127 magnitudes.

    Scans the table of non-negative magnitudes; on an exact tie between two
    neighbours it takes the one whose code is even (even mantissa).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("|v| > 448")
    table = e4m3_values()
    a = np.abs(v).ravel()
    hi = np.searchsorted(table, a, side="left")          # first table >= a
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(table[hi] == a, hi, pick)
    code = pick.astype(np.int64) | (np.signbit(v.ravel()).astype(np.int64) << 7)
    return code.astype(np.uint8).reshape(v.shape)


def bf16_round(v):
    """Round float64 values to the nearest bfloat16 (ties to even), once.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
    exponent range.  Returns the rounded values as float64 together with the
    16-bit patterns (uint16).  Rounding straight from float64 avoids the
    double rounding float64 -> float32 -> bf16 would introduce.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)):
        raise ValueError("bf16_round expects finite input")
    f, ex = np.frexp(np.abs(v))              # |v| = f * 2^ex, f in [0.5, 1)
    ex = np.maximum(ex, -125)                # below 2^-126 the spacing is fixed (subnormals)
    spacing = np.exp2(ex.astype(np.float64) - 8.0)
    r = np.rint(np.abs(v) / spacing) * spacing
    r = np.where(np.signbit(v), -r, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return r, bits
