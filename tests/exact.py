"""Exact (rational / integer) arithmetic used to pin the oracle.

Nothing here shares code with ``oracle/``: bf16 / fp16 patterns are decoded
into integers by hand and rounding is done on Python integers, so a slip in
the oracle's float-based helpers cannot hide behind the same slip here.
"""

from fractions import Fraction

import numpy as np


def bf16_fraction(b):
    """bf16 bit pattern -> exact Fraction (finite only)."""
    b = int(b)
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    assert e != 0xFF
    if e == 0:
        v = Fraction(m, 1 << 133)
    else:
        v = Fraction(m + 128) * (Fraction(2) ** (e - 127 - 7))
    return sign * v


def f16_fraction(b):
    b = int(b)
    sign = -1 if b & 0x8000 else 1
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    assert e != 0x1F
    if e == 0:
        v = Fraction(m, 1 << 24)
    else:
        v = Fraction(m + 1024) * (Fraction(2) ** (e - 15 - 10))
    return sign * v


def _floor_log2(a):
    """floor(log2(a)) for a positive Fraction."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _rne_int(x):
    """Round a non-negative Fraction to the nearest integer, ties to even."""
    n = x.numerator // x.denominator
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def rne_fraction(v, p, qmin, emax):
    """Exact round-to-nearest-even of a Fraction onto a binary format grid:
    returns a Fraction, or +-inf as float."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = _floor_log2(a)
    q = max(e - (p - 1), qmin)
    r = _rne_int(a / (Fraction(2) ** q))
    res = r * (Fraction(2) ** q)
    if res >= Fraction(2) ** (emax + 1):
        return float("inf") if v > 0 else float("-inf")
    return res if v > 0 else -res


def rne_bf16_fraction(v):
    return rne_fraction(v, 8, -133, 127)


def rne_fp16_fraction(v):
    return rne_fraction(v, 11, -24, 15)


def fraction_to_bf16_bits(v):
    """Exact bf16 value (Fraction, or +-inf) -> bit pattern.  Zero -> +0."""
    if isinstance(v, float):
        return 0x7F80 if v > 0 else 0xFF80
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return 0
    e = _floor_log2(a)
    if e < -126:
        m = a * (Fraction(2) ** 133)
        assert m.denominator == 1 and m < 128
        return sign | int(m)
    m = a / (Fraction(2) ** (e - 7))
    assert m.denominator == 1 and 128 <= m < 256
    return sign | ((e + 127) << 7) | (int(m) - 128)


def bf16_int_parts(bits):
    """Vectorised: bf16 bits -> (signed integer significand W, exponent a) with
    value = W * 2**a exactly (zeros give W = 0)."""
    b = np.asarray(bits, dtype=np.int64)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    sig = np.where(e == 0, m, m + 128)
    a = np.where(e == 0, -133, e - 127 - 7)
    sig = np.where(b & 0x8000, -sig, sig)
    return sig, a


def _scaled_ints(sig, a, shift):
    """Python integers sig * 2**(a + shift) (exact; a + shift >= 0)."""
    sig = np.asarray(sig, dtype=object)
    e = np.asarray(a + shift, dtype=np.int64)
    assert np.all(e >= 0)
    return sig * np.vectorize(lambda t: 1 << int(t), otypes=[object])(e)


def f16_int_parts(bits):
    """Vectorised: fp16 bits -> (signed integer significand, exponent) with
    value = sig * 2**a exactly (zeros give 0).  Infinities are not decoded:
    callers replace them."""
    b = np.asarray(bits, dtype=np.int64)
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    sig = np.where(e == 0, m, m + 1024)
    a = np.where(e == 0, -24, e - 15 - 10)
    sig = np.where(b & 0x8000, -sig, sig)
    return sig, a


def nearest_int_argmin(x_int, lev_int):
    """Lowest index of the smallest |x - v| on Python integers.
    x_int [..., G], lev_int [..., L] (object arrays) -> int64 [..., G]."""
    d = np.abs(x_int[..., :, None] - lev_int[..., None, :])
    return np.argmin(d, axis=-1).astype(np.int64)


# Every bf16 value times 2**133 and every product of two bf16 values times
# 2**266 is an integer; fp16 values times 2**24 are integers.
BIG_INF = 1 << 2000   # stands for +inf: farther than any finite level


def lut16_exact_indices(w_bits, s_bits, lut_bits):
    """Brute-force exact nearest level of LUT16 on integers: w [rows, 64],
    s [rows, 1], L [rows, 1, 16] (one group per row)."""
    ws, wa = bf16_int_parts(w_bits)
    X = _scaled_ints(ws, wa, 266)                                     # w * 2**266
    ss, sa = bf16_int_parts(np.asarray(s_bits)[:, 0])
    ls, la = bf16_int_parts(np.asarray(lut_bits)[:, 0, :])
    V = _scaled_ints(ss[:, None] * ls, sa[:, None] + la, 266)         # s L * 2**266
    return nearest_int_argmin(X, V)


def signmag8_exact_indices(w_bits, cb_bits):
    """Brute-force exact sign + nearest magnitude on integers: w [rows, 64]
    (two groups of 32 per row), cb [rows, 2, 8] fp16 bits (+inf allowed)."""
    w_bits = np.asarray(w_bits)
    rows = w_bits.shape[0]
    ws, wa = bf16_int_parts(w_bits)
    A = np.abs(_scaled_ints(ws, wa, 133)).reshape(rows, 2, 32)        # |w| * 2**133
    cb = np.asarray(cb_bits)
    ms, ma = f16_int_parts(cb)
    M = _scaled_ints(ms, ma, 133)                                     # M * 2**133
    M = np.where(cb == 0x7C00, BIG_INF, M)
    mag = nearest_int_argmin(A, M).reshape(rows, 64)
    neg = ((w_bits & 0x8000) != 0) & ((w_bits & 0x7FFF) != 0)   # w < 0 (-0.0 is not)
    return (mag | np.where(neg, 8, 0)).astype(np.uint8)
