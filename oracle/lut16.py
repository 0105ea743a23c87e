"""Per-group 16-entry LUT codec (1D k-means levels), group 64.

Oracle (test infrastructure).  K-means page:

* section 1.2: every block of 64 weights gets its own 1D k-means clustering
  with N = 2**n_bits = 16 centres plus a 16-bit scale; the index of a weight
  is its nearest centre (``nearest_neighbor``);
* section 2.2: decode is a table lookup of the precomputed outputs for the 16
  possible 4-bit indices.

Format (one reading, listed in the design notes): per group a bf16 scale
``s`` (the group's absmax) and 16 bf16 normalised levels ``L_j`` in [-1, 1];
the group's levels are the exact products ``v_j = s * L_j`` (8 x 8
significant bits) and the reconstructed weight is ``RNE_bf16(v_idx)``.

The index of a weight is the lowest j minimising the exact distance
``|w - v_j|`` (``oracle.nearest``), for every finite weight, scale and table:
also for weights far outside the levels' range and for tables whose levels
are far apart in magnitude, where a distance rounded to fp32 or fp64 no
longer separates the levels.

The fit (used only to make test data) is the k-means page's per-block 1D
k-means with the seeding and iteration count that the int4-g32 page
describes for its Lloyd step (section 1.3: quantile start, 25 rounds):
normalise ``u = w / s`` in fp64, start from ``c_k = sorted(u)[4k + 2]``,
then 25 rounds of (assign each u to its nearest centre, ties to the lower
centre; move each centre to the fp64 mean of its members summed in
increasing element order; an empty centre stays put), and finally
``L_k = RNE_bf16(c_k)``.  The fitted centres are pinned only by procedure
(monotone MSE, exact recovery of 16-point data, agreement with the C
implementation, never below the optimal 1D k-means cost): their exact values
are "parity unpinned".
"""

import numpy as np

from .bits import bf16_to_f64, f32_to_bf16_bits_exact, rne_bf16
from .nearest import nearest
from .packing import pack, unpack

GROUP = 64
N_LEVELS = 16
LLOYD_ITERS = 25


def levels(s_bits, lut_bits):
    """Group levels ``v_j = s * L_j`` as fp64 (exact: at most 16 significant
    bits, exponents between -266 and 255).  s [N, G], L [N, G, 16]."""
    s = bf16_to_f64(s_bits)[..., None]
    L = bf16_to_f64(lut_bits)
    return s * L


def indices(w_bits, s_bits, lut_bits, chunk_rows=256):
    """Exact nearest level, lowest index on ties; w [N, K] -> idx uint8 [N, K]."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    g = k // GROUP
    out = np.empty((n, k), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        w = bf16_to_f64(w_bits[r0:r1]).reshape(r1 - r0, g, GROUP)
        v = levels(s_bits[r0:r1], lut_bits[r0:r1])                     # [r, G, 16]
        out[r0:r1] = nearest(w, v).astype(np.uint8).reshape(r1 - r0, k)
    return out


def quantize_pack(w_bits, s_bits, lut_bits):
    """w bf16 bits [N, K] with a given (scale, LUT) -> packed uint8 [N, K/2]."""
    return pack(indices(w_bits, s_bits, lut_bits))


def dequant_from_indices(idx, s_bits, lut_bits):
    """bf16 bits of ``RNE_bf16(s * L[idx])`` (sign of a zero product kept)."""
    idx = np.asarray(idx)
    n, k = idx.shape
    g = k // GROUP
    L = bf16_to_f64(lut_bits)                                   # [N, G, 16]
    sel = np.take_along_axis(L, idx.reshape(n, g, GROUP).astype(np.int64), axis=-1)
    v = bf16_to_f64(s_bits)[..., None] * sel                    # exact product
    return rne_bf16(v).reshape(n, k)


def dequant(packed, s_bits, lut_bits):
    return dequant_from_indices(unpack(packed), s_bits, lut_bits)


# ----------------------------------------------------------------- fit (test data)
def quantile_init(u, n_levels):
    """``c_k = sorted(u)[k * (G / n) + (G / n) // 2]`` for each row of u [B, G].

    The sort is stable: equal values (also -0.0 and +0.0) keep their element
    order, so the start is fully determined by the group."""
    gsz = u.shape[-1]
    stride = gsz // n_levels
    srt = np.sort(u, axis=-1, kind="stable")
    return srt[..., stride * np.arange(n_levels) + stride // 2].copy()


def lloyd(u, c, iters=LLOYD_ITERS, history=False):
    """1D Lloyd / k-means on each row of u [B, G] from centres c [B, n].

    Assignment: nearest centre by |u - c| in fp64, lowest centre index on a
    tie.  Update: fp64 sum of the members in increasing element order, divided
    by the member count; a centre with no members keeps its value."""
    u = np.asarray(u, dtype=np.float64)
    c = np.array(c, dtype=np.float64)
    n = c.shape[-1]
    ks = np.arange(n)
    mses = []
    for _ in range(iters):
        a = np.argmin(np.abs(u[..., :, None] - c[..., None, :]), axis=-1)   # [B, G]
        if history:
            mses.append(np.mean((u - np.take_along_axis(c, a, axis=-1)) ** 2, axis=-1))
        sums = np.zeros_like(c)
        cnt = np.zeros(c.shape, dtype=np.int64)
        for i in range(u.shape[-1]):                 # members in increasing order
            hit = a[..., i, None] == ks
            sums = sums + np.where(hit, u[..., i, None], 0.0)
            cnt = cnt + hit
        c = np.where(cnt > 0, sums / np.maximum(cnt, 1), c)
    if history:
        a = np.argmin(np.abs(u[..., :, None] - c[..., None, :]), axis=-1)
        mses.append(np.mean((u - np.take_along_axis(c, a, axis=-1)) ** 2, axis=-1))
        return c, np.stack(mses, axis=-1)
    return c


def fit(w_bits, iters=LLOYD_ITERS):
    """k-means LUT fit.  w [N, K] -> (scale bits [N, K/64], LUT bits [N, K/64, 16])."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    g = k // GROUP
    w = bf16_to_f64(w_bits).reshape(n * g, GROUP)
    s = np.max(np.abs(w), axis=-1)
    safe = np.where(s == 0.0, 1.0, s)
    u = w / safe[:, None]
    c = lloyd(u, quantile_init(u, N_LEVELS), iters)
    c = np.where((s == 0.0)[:, None], 0.0, c)
    s_bits = f32_to_bf16_bits_exact(s.astype(np.float32)).reshape(n, g)
    return s_bits, rne_bf16(c).reshape(n, g, N_LEVELS)


# ----------------------------------------------------------------- LUT16S
# One 16-level table for the whole weight plus a bf16 scale (the group's
# absmax) per group of 64: the reading of the k-means page under which its
# 3.9B model takes about 2.1 GB (section 2.1; 4.25 bits per weight).  The
# rebuild and the nearest-level rule are LUT16's with that table in every
# group.

def group_scales(w_bits):
    """Group absmax as bf16 bits [N, K/64] (exact: the absmax is a bf16 value)."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    w = bf16_to_f64(w_bits).reshape(n, k // GROUP, GROUP)
    s = np.max(np.abs(w), axis=-1)
    return f32_to_bf16_bits_exact(s.astype(np.float32))


def shared_tables(s_bits, table_bits):
    """The one table [16] repeated for every group: [N, K/64, 16]."""
    return np.broadcast_to(np.asarray(table_bits, dtype=np.uint16), s_bits.shape + (N_LEVELS,))


def fit_shared(w_bits, iters=LLOYD_ITERS):
    """Whole-weight k-means table.  w [N, K] -> (scale bits [N, K/64], table bits [16]).

    u = w / s per group (fp64; an all-zero group gives zeros); the start is
    ``sorted(u)[q * (T/16) + T/32]`` over all T = N*K values of u in row-major
    element order (stable sort); then `iters` Lloyd rounds exactly as in the
    per-group fit, over all of u at once: nearest centre with the lowest index
    on ties, each centre moved to the fp64 sum of its members in increasing
    element order divided by their count, an empty centre kept.  Levels are
    ``RNE_bf16(c)``.  Test-data generator: parity unpinned beyond the
    procedure pins (it equals the per-group fit on a one-group weight)."""
    w_bits = np.asarray(w_bits)
    n, k = w_bits.shape
    s_bits = group_scales(w_bits)
    w = bf16_to_f64(w_bits).reshape(n, k // GROUP, GROUP)
    s = bf16_to_f64(s_bits)[..., None]
    u = (w / np.where(s == 0.0, 1.0, s)).reshape(-1)
    t = u.size
    stride = t // N_LEVELS
    c = np.sort(u, kind="stable")[stride * np.arange(N_LEVELS) + stride // 2].copy()
    for _ in range(iters):
        a = np.empty(t, dtype=np.int64)
        for i0 in range(0, t, 1 << 20):                  # assignment in chunks
            d = np.abs(u[i0:i0 + (1 << 20), None] - c[None, :])
            a[i0:i0 + (1 << 20)] = np.argmin(d, axis=-1)
        sums = np.bincount(a, weights=u, minlength=N_LEVELS)  # one pass in element order
        cnt = np.bincount(a, minlength=N_LEVELS)
        c = np.where(cnt > 0, sums / np.maximum(cnt, 1), c)
    return s_bits, rne_bf16(c)


# ----------------------------------------------------------------- LUT16S_IL
# The k-means page (section 2.2) suggests storing the scales with the indices
# so that one read brings both.  Layout only, no arithmetic: per row and
# 256-k block, a 144-byte record of the block's 128 packed bytes, its four
# bf16 scales (little-endian) and 8 zero bytes.

IL_RECORD = 144


def interleave(packed, s_bits):
    """packed uint8 [N, K/2], scale bits [N, K/64] (K % 256 == 0) -> uint8 [N, K/256 * 144]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape
    nb = 2 * half // 256
    out = np.zeros((n, nb, IL_RECORD), np.uint8)
    out[:, :, :128] = packed.reshape(n, nb, 128)
    sc = np.ascontiguousarray(np.asarray(s_bits, dtype="<u2").reshape(n, nb, 4))
    out[:, :, 128:136] = sc.view(np.uint8).reshape(n, nb, 8)
    return out.reshape(n, nb * IL_RECORD)


def deinterleave(il):
    """Inverse of interleave: uint8 [N, K/256 * 144] -> (packed [N, K/2], scale bits [N, K/64])."""
    il = np.asarray(il, dtype=np.uint8)
    n = il.shape[0]
    rec = il.reshape(n, -1, IL_RECORD)
    packed = np.ascontiguousarray(rec[:, :, :128]).reshape(n, -1)
    s_bits = np.ascontiguousarray(rec[:, :, 128:136]).view("<u2").reshape(n, -1).astype(np.uint16)
    return packed, s_bits
