"""Two 4-bit indices per byte.

Oracle (test infrastructure).  DyadicGumbel page, section 2.5: after the hard
argmin each 4-bit index sits in a uint8, and two indices are packed into one
byte as ``lo | hi << 4``.  Reading taken where the page is silent: along a
row, element ``2j`` goes into the low nibble of byte ``j`` and element
``2j+1`` into the high nibble.

Pinned by the round trip over all 256 byte values and by hand-derived bytes in
``tests/golden/packing_examples.txt``.
"""

import numpy as np


def pack(idx):
    """idx uint8 [..., K] with values 0..15, K even -> packed uint8 [..., K/2]."""
    idx = np.asarray(idx)
    if idx.shape[-1] % 2:
        raise ValueError("K must be even")
    if idx.size and (idx.min() < 0 or idx.max() > 15):
        raise ValueError("indices must be in 0..15")
    lo = idx[..., 0::2].astype(np.uint8)
    hi = idx[..., 1::2].astype(np.uint8)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack(packed):
    """packed uint8 [..., K/2] -> idx uint8 [..., K]."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0x0F)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def storage_bytes(n_weights, group, scale_bytes_per_group):
    """Bytes of a packed weight with a per-group side table: n/2 for the
    nibbles plus ``scale_bytes_per_group`` per group (DyadicGumbel page,
    section 2.5: 679M x 4 bit / 8 = 340 MB plus 21 MB of bf16 scales)."""
    n_groups = -(-n_weights // group)
    return n_weights // 2 + n_groups * scale_bytes_per_group
