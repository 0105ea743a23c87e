"""Bit patterns of the storage types, and correct rounding into them.

Oracle (test infrastructure).  The weights, scales and LUT entries on the
DyadicGumbel page (section 2.2, "scale_i (bf16)") and the k-means page
(section 1.2, 16-bit per-block scale) are bf16; the int4-g32 page's dense
inference weight (section 2, "稠密 fp16 权重") is fp16.  This module holds
those formats and nothing of the method.

``rne_bf16`` / ``rne_fp16`` round an fp64 value to the nearest representable
value with ties to even (IEEE 754 roundTiesToEven), including the subnormal
range and overflow to infinity.  They are written from the definition of the
format: a finite value is ``integer * 2**q`` where the quantum exponent ``q``
is ``e - (p - 1)`` for a value in ``[2**e, 2**(e+1))`` with ``p`` significant
bits, but never below the subnormal quantum.  Pinned against exact rational
rounding and against an independent bit-level method in
``tests/test_oracle_bits.py``.
"""

import numpy as np

# bf16: 8 significant bits, smallest normal exponent -126 -> subnormal quantum 2**-133
BF16_P, BF16_QMIN, BF16_EMAX = 8, -133, 127
# fp16: 11 significant bits, smallest normal exponent -14 -> subnormal quantum 2**-24
FP16_P, FP16_QMIN, FP16_EMAX = 11, -24, 15


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits):
    """fp16 bit patterns (uint16) -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_bf16_bits_exact(x32):
    """float32 values that are exactly representable in bf16 -> bf16 bits.

    Raises if any value would need rounding (used for values that are bf16 by
    construction, e.g. an absmax of bf16 inputs)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value not exactly representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


def _round_to_grid(x, p, qmin, emax):
    """Round |x| (fp64) to the grid of a binary format with ``p`` significant
    bits, subnormal quantum 2**qmin and largest finite exponent ``emax``;
    returns (magnitude as fp64 or inf, sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("finite inputs only")
    sign = np.signbit(x)
    a = np.abs(x)
    _, E = np.frexp(a)            # a = m * 2**E with m in [0.5, 1); e = E - 1
    e = E.astype(np.int64) - 1
    q = np.maximum(e - (p - 1), qmin)
    r = np.rint(np.ldexp(a, -q))  # exact scaling by a power of two, then ties-to-even
    mag = np.ldexp(r, q)
    mag = np.where(a == 0.0, 0.0, mag)
    # overflow: a rounded magnitude of 2**(emax+1) or more is infinity
    mag = np.where(mag >= np.ldexp(1.0, emax + 1), np.inf, mag)
    return mag, sign


def rne_bf16(x):
    """Round fp64 values to bf16 (ties to even); returns uint16 bit patterns.
    The sign of zero is kept."""
    mag, sign = _round_to_grid(x, BF16_P, BF16_QMIN, BF16_EMAX)
    with np.errstate(over="ignore"):
        u = mag.astype(np.float32).view(np.uint32) >> np.uint32(16)
    u = u.astype(np.uint16)
    return np.where(sign, u | np.uint16(0x8000), u).astype(np.uint16)


def rne_fp16(x):
    """Round fp64 values to fp16 (ties to even); returns uint16 bit patterns.
    The sign of zero is kept."""
    mag, sign = _round_to_grid(x, FP16_P, FP16_QMIN, FP16_EMAX)
    with np.errstate(over="ignore"):
        u = mag.astype(np.float16).view(np.uint16)
    return np.where(sign, u | np.uint16(0x8000), u).astype(np.uint16)


def all_finite_bf16():
    """Every finite bf16 bit pattern (both signs, both zeros)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (b >> np.uint16(7)) & np.uint16(0xFF)
    return b[exp != 0xFF]
