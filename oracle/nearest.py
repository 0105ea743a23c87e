"""Exact nearest level with the lowest index on ties.

Oracle (test infrastructure).  The k-means page (section 1.2) gives every
weight the index of its nearest centre; the int4-g32 page (section 1.3, step
4) gives every magnitude its nearest level.  Neither says how ties or
rounding are handled; the reading here is the exact one: the index is the
lowest j minimising the exact real distance |x - v_j|.

Inputs are fp64 arrays that hold their values exactly: bf16 weights or
magnitudes, products of two bf16 numbers (at most 16 significant bits and an
exponent inside the fp64 normal range), fp16 magnitudes, and +inf (an fp16
magnitude that overflowed).  The computation has two steps:

1. ``d_j = fl64(|x - v_j|)``.  Correct rounding is monotone, so a level whose
   rounded distance is strictly larger than the smallest rounded distance is
   also strictly farther in exact arithmetic, and the exact nearest level is
   among those that share the smallest rounded distance.
2. Where two or more levels share that smallest rounded distance, the exact
   distances of those levels are compared in rational arithmetic
   (``fractions.Fraction``, exact for every finite float).  If the smallest
   rounded distance is +inf, every level is +inf away and the lowest index
   is the answer.
"""

from fractions import Fraction

import numpy as np


def nearest(x, levels):
    """x [..., G] (fp64), levels [..., L] (fp64, the same leading shape) ->
    index [..., G] (int64) of the lowest level at the smallest exact distance."""
    x = np.asarray(x, dtype=np.float64)
    levels = np.asarray(levels, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        d = np.abs(x[..., :, None] - levels[..., None, :])          # [..., G, L]
    idx = np.argmin(d, axis=-1)                                       # first rounded minimum
    dmin = np.take_along_axis(d, idx[..., None], axis=-1)
    tied = (d == dmin) & np.isfinite(dmin)
    several = np.count_nonzero(tied, axis=-1) > 1
    if np.any(several):
        lev = np.broadcast_to(levels[..., None, :], d.shape)
        xs = np.broadcast_to(x[..., None], d.shape)
        for pos in zip(*np.nonzero(several)):
            cand = np.flatnonzero(tied[pos])
            xv = Fraction(float(xs[pos][0]))
            exact = [abs(xv - Fraction(float(lev[pos][j]))) for j in cand]
            best = min(exact)
            idx[pos] = int(cand[exact.index(best)])
    return idx
