"""Dyadic 4-bit codec, group 64 along the input dimension.

Oracle (test infrastructure).  DyadicGumbel page:

* section 2.1: with b = 4 bits, ``half = 2**(b-1) = 8``, ``step = scale/half``
  and the codebook is ``step * {-8, -7, ..., 7}`` -- 16 equally spaced values;
* section 2.2: each layer is cut into blocks of ``group_size = 64`` weights;
  block i stores ``scale_i`` (bf16, the codebook's half range) and 64 4-bit
  level indices; reconstruction is ``w[j] = step_i * (level_idx[j] - half)``;
* sections 2.3 / 2.5: the index is the hard argmin of the distance from the
  weight to the codebook entries.

Readings taken where the page is silent (each listed in the design notes):

* a group is 64 consecutive weights along K of the row-major [N, K] weight;
* the scale is the group's absolute maximum (the zero-shot / post-training
  reading of "codebook half range"); it is itself a bf16 value, exactly;
* distance is ``|w - code|`` against the exact codes (no rounding of the
  codes), the lowest index wins a tie;
* an all-zero group gets scale +0 and index 8 everywhere (so index 8 always
  means 0), rather than the tie rule's index 0;
* the reconstructed value is the exact product rounded once to bf16 (ties to
  even), and a zero result is +0.
"""

import numpy as np

from .bits import bf16_to_f64, f32_to_bf16_bits_exact, rne_bf16
from .packing import pack, unpack

GROUP = 64
HALF = 8          # 2**(4-1)
N_LEVELS = 16


def _grouped(a, group=GROUP):
    a = np.asarray(a)
    n, k = a.shape
    if k % group:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    return a.reshape(n, k // group, group)


def scales(w_bits):
    """Per-group absmax scale.  w bf16 bits [N, K] -> scale bf16 bits [N, K/64]."""
    w = bf16_to_f64(_grouped(w_bits))
    s = np.max(np.abs(w), axis=-1)
    return f32_to_bf16_bits_exact(s.astype(np.float32))


def codebook(s):
    """Exact codes ``(s/8) * (j - 8)``, j = 0..15, for fp64 scales s [...] -> [..., 16]."""
    j = np.arange(N_LEVELS, dtype=np.float64)
    return (np.asarray(s, dtype=np.float64)[..., None] / HALF) * (j - HALF)


def indices(w_bits, s_bits, chunk_rows=256):
    """Hard argmin: for each weight the smallest j minimising ``|w - c_j|``.

    Written as the definition: all 16 distances in fp64, first minimum.  (The
    distances are exact in fp64 whenever |w| >= s * 2**-46; below that the
    nearest code is 0 by a margin no rounding can close.)"""
    w_bits = np.asarray(w_bits)
    s_bits = np.asarray(s_bits)
    n, k = w_bits.shape
    out = np.empty((n, k), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        w = bf16_to_f64(_grouped(w_bits[r0:r0 + chunk_rows]))      # [r, G, 64]
        s = bf16_to_f64(s_bits[r0:r0 + chunk_rows])                 # [r, G]
        c = codebook(s)                                             # [r, G, 16]
        dist = np.abs(w[..., :, None] - c[..., None, :])            # [r, G, 64, 16]
        idx = np.argmin(dist, axis=-1).astype(np.uint8)             # first minimum
        idx = np.where((s == 0.0)[..., None], np.uint8(HALF), idx)  # all-zero group
        out[r0:r0 + chunk_rows] = idx.reshape(idx.shape[0], k)
    return out


def quantize_pack(w_bits):
    """w bf16 bits [N, K] -> (packed uint8 [N, K/2], scale bf16 bits [N, K/64])."""
    s = scales(w_bits)
    return pack(indices(w_bits, s)), s


def dequant_from_indices(idx, s_bits):
    """idx [N, K], scale bits [N, K/64] -> bf16 bits of ``RNE((s/8)*(idx-8))``."""
    idx = _grouped(idx).astype(np.float64)
    s = bf16_to_f64(s_bits)[..., None]
    v = (s / HALF) * (idx - HALF)      # exact in fp64 (<= 11 significant bits)
    v = np.where(v == 0.0, 0.0, v)     # a zero result is +0
    out = rne_bf16(v)
    return out.reshape(out.shape[0], -1)


def dequant(packed, s_bits):
    """packed [N, K/2], scale bits [N, K/64] -> dense bf16 bits [N, K]."""
    return dequant_from_indices(unpack(packed), s_bits)
