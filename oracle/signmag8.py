"""Sign + 3-bit magnitude codec with a per-group 8-level fp16 codebook, group 32.

Oracle (test infrastructure).  int4-g32 page:

* section 1.1: the weight matrix is cut along the input dimension into groups
  of 32 and each group is handled on its own;
* section 1.3 (step 4): ``|w~| = nearest level``, ``w~ = sign * |w~|``, the
  sign kept separately in one bit;
* section 2: per weight 4 bits = 3-bit level index (0..7, magnitude) + 1 sign
  bit; at inference the weights are rebuilt to a dense fp16 matrix by a
  per-group lookup of (level table, sign).

Readings (listed in the design notes): the group's 8 magnitudes are stored
as fp16 (the page's 8-bit parameter code that regenerates a parametric table
is not stored; the Lloyd-refined levels are); inside the nibble bit 3 is the
sign and bits 0..2 the magnitude index; the sign bit is ``w < 0`` (so -0.0
gets sign 0); the magnitude index is the lowest j minimising the exact
distance ``||w| - M_j|`` (``oracle.nearest``; a magnitude of +inf, which the
fit produces for groups beyond the fp16 range, is infinitely far from every
finite weight); dequant is exactly ``±M[mag]`` in fp16 (so sign 1 with M = 0
gives -0.0).

The fit (test data only) is the page's "cold start" (section 1.4: quantile
initial levels, then Lloyd): ``c_k = sorted(|w|)[4k + 2]``, 25 Lloyd rounds
in fp64, ``M_k = RNE_fp16(c_k)``.  Its exact output is "parity unpinned"
(pinned by procedure, as for the LUT16 fit).
"""

import numpy as np

from .bits import bf16_to_f64, f16_to_f64, rne_fp16
from .lut16 import lloyd, quantile_init, LLOYD_ITERS
from .nearest import nearest
from .packing import pack, unpack

GROUP = 32
N_MAG = 8


def indices(w_bits, cb_bits, chunk_rows=256):
    """w bf16 bits [N, K], codebook fp16 bits [N, K/32, 8] -> nibbles uint8 [N, K]."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    g = k // GROUP
    out = np.empty((n, k), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        w = bf16_to_f64(w_bits[r0:r1]).reshape(r1 - r0, g, GROUP)
        m = f16_to_f64(cb_bits[r0:r1])                                  # [r, G, 8]
        mag = nearest(np.abs(w), m).astype(np.uint8)
        sign = (w < 0).astype(np.uint8)
        out[r0:r1] = ((sign << 3) | mag).reshape(r1 - r0, k)
    return out


def quantize_pack(w_bits, cb_bits):
    return pack(indices(w_bits, cb_bits))


def dequant_from_indices(nib, cb_bits):
    """nibbles [N, K] -> fp16 bits [N, K] of ``±M[nib & 7]`` (exact)."""
    nib = np.asarray(nib)
    n, k = nib.shape
    g = k // GROUP
    nb = nib.reshape(n, g, GROUP).astype(np.int64)
    m = np.take_along_axis(np.asarray(cb_bits, dtype=np.uint16), nb & 7, axis=-1)
    sign = ((nb >> 3) & 1).astype(np.uint16) << np.uint16(15)
    return (m ^ sign).astype(np.uint16).reshape(n, k)


def dequant(packed, cb_bits):
    return dequant_from_indices(unpack(packed), cb_bits)


def fit(w_bits, iters=LLOYD_ITERS):
    """Cold-start Lloyd fit of the 8 magnitudes.  w [N, K] -> fp16 bits [N, K/32, 8]."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    g = k // GROUP
    a = np.abs(bf16_to_f64(w_bits)).reshape(n * g, GROUP)
    c = lloyd(a, quantile_init(a, N_MAG), iters)
    return rne_fp16(c).reshape(n, g, N_MAG)


def dequant_values(cb_bits, nib):
    """fp64 values of the dequantized weights (for the matmul reference)."""
    return f16_to_f64(dequant_from_indices(nib, cb_bits))
