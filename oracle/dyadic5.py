"""Dyadic codec with 3-, 4- and 5-bit groups in one 5-bit index space.

Oracle (test infrastructure).  DyadicGumbel page, section 2.1: with b bits,
``half = 2**(b-1)``, ``step = scale/half`` and the codes are
``step * {-half, ..., half-1}``; the page notes that the 3-, 4- and 5-bit
codebooks share one level index space, so that a block's precision can change
without rebuilding the codebook (its "water-filling", section 6, left off).

Reading (listed in the design notes): the codes nest -- the b-bit code j is
the 5-bit code ``j * 2**(5-b)`` -- so every group is stored as 5-bit indices
``j5`` with value ``(s/16) * (j5 - 16)``, and a group's width b in {3, 4, 5}
only restricts which codes its weights may take.  The page gives no rule for
choosing the widths; they are an input.

* scale: the group's absmax (a bf16 value), as for the 4-bit codec;
* index: among the group's b-bit codes, the lowest j minimising ``|w - c_j|``
  against the exact codes; an all-zero group gets the zero code (j5 = 16);
* rebuild: ``RNE_bf16((s/16) * (j5 - 16))``; an exact zero product is +0, a
  nonzero product that rounds to zero keeps its sign.

Storage of j5 for an [N, K] weight (the format the library reads and writes):
* nibble plane uint8 [N, K/2]: ``j5 & 15`` packed two per byte like the 4-bit
  codec (element 2c in the low nibble);
* high-bit plane uint8 [N, K/8]: per run of 32 weights (k = 32c .. 32c+31) one
  little-endian 32-bit word M holding ``j5 >> 4`` of weight 32c + i at bit
  ``msb_bit(i)`` below.
"""

import numpy as np

from .bits import bf16_to_f64, rne_bf16
from .dyadic import scales
from .packing import pack, unpack

GROUP = 64
WIDTHS = (3, 4, 5)

# bit of the 32-bit word M that holds the high bit of weight i (0..31) of its
# run of 32: weight i sits in packed dword d = i // 8 at position e = i % 8;
# positions (0, 4), (1, 5), (2, 6), (3, 7) form the dword's four value pairs,
# whose high bits sit at bits (4, 20), (8, 24), (4, 20), (8, 24) of a word
# taken from M shifted by SHIFT[2d] for the first two pairs and SHIFT[2d + 1]
# for the last two.
_PAIR_BIT = (4, 8, 4, 8, 20, 24, 20, 24)
SHIFT = (-4, -3, -2, -1, 4, 5, 6, 7)


def msb_bit(i):
    d, e = divmod(i, 8)
    t = 2 * d + (1 if (e % 4) >= 2 else 0)
    return _PAIR_BIT[e] + SHIFT[t]


def _grouped(a):
    a = np.asarray(a)
    n, k = a.shape
    if k % GROUP:
        raise ValueError(f"K={k} is not a multiple of the group size {GROUP}")
    return a.reshape(n, k // GROUP, GROUP)


def indices(w_bits, s_bits, widths=None):
    """5-bit indices [N, K] for bf16 weights with given scales and group widths
    (uint8 [N, K/64]; 3 and 4 select those widths, any other value 5; None:
    all 5).  Written as the definition:
    every code's distance in fp64, first minimum (the distances are exact in
    fp64 unless |w| < s * 2**-45, where code 0 wins by a margin no rounding
    can close)."""
    w = bf16_to_f64(_grouped(w_bits))                       # [N, G, 64]
    s = bf16_to_f64(np.asarray(s_bits))                     # [N, G]
    n, g, _ = w.shape
    if widths is None:
        widths = np.full((n, g), 5, dtype=np.uint8)
    widths = np.asarray(widths)
    widths = np.where((widths == 3) | (widths == 4), widths, 5)
    out = np.empty((n, g, GROUP), dtype=np.uint8)
    for b in WIDTHS:
        half = 2 ** (b - 1)
        sel = widths == b
        if not sel.any():
            continue
        ws, ss = w[sel], s[sel]                             # [M, 64], [M]
        codes = (ss[:, None] / half) * (np.arange(2 * half) - half)   # exact
        j = np.argmin(np.abs(ws[:, :, None] - codes[:, None, :]), axis=-1)
        j = np.where((ss == 0.0)[:, None], half, j)         # all-zero group
        out[sel] = (j * 2 ** (5 - b)).astype(np.uint8)
    return out.reshape(n, g * GROUP)


def quantize(w_bits, widths=None):
    """-> (5-bit indices [N, K], scale bits [N, K/64])."""
    s = scales(w_bits)
    return indices(w_bits, s, widths), s


def planes(idx5):
    """5-bit indices [N, K] -> (nibble plane [N, K/2], high-bit plane [N, K/8])."""
    idx5 = np.asarray(idx5, dtype=np.uint32)
    n, k = idx5.shape
    runs = (idx5 >> 4).reshape(n, k // 32, 32)
    words = np.zeros((n, k // 32), dtype=np.uint32)
    for i in range(32):
        words |= runs[:, :, i] << np.uint32(msb_bit(i))
    return pack((idx5 & 15).astype(np.uint8)), words.astype("<u4").view(np.uint8).reshape(n, k // 8)


def unplanes(nibbles, msb):
    """Inverse of planes."""
    lo = unpack(nibbles).astype(np.uint32)
    n, k = lo.shape
    words = np.ascontiguousarray(msb).view("<u4").reshape(n, k // 32).astype(np.uint32)
    hi = np.empty((n, k // 32, 32), dtype=np.uint32)
    for i in range(32):
        hi[:, :, i] = (words >> np.uint32(msb_bit(i))) & 1
    return (lo | (hi.reshape(n, k) << 4)).astype(np.uint8)


def dequant_from_indices(idx5, s_bits):
    """bf16 bits of ``RNE_bf16((s/16) * (j5 - 16))``."""
    j = _grouped(idx5).astype(np.float64)
    s = bf16_to_f64(np.asarray(s_bits))[..., None]
    v = (s / 16.0) * (j - 16.0)        # exact in fp64 (<= 13 significant bits)
    v = np.where(v == 0.0, 0.0, v)     # an exact zero is +0
    out = rne_bf16(v)
    return out.reshape(out.shape[0], -1)


def dequant(nibbles, msb, s_bits):
    return dequant_from_indices(unplanes(nibbles, msb), s_bits)
