"""Exhaustive quantize sweeps shared by the CPU pins of the oracle and the GPU
parity tests, so that the checker the GPU tests use (``oracle/liboracle.c``)
is pinned on exactly the inputs it judges.

Every case holds every finite bf16 weight (both signs, both zeros), laid out
in rows of one group's width or more, together with side data at the edges
of what the library accepts: scales from the smallest subnormal to the
largest finite bf16, tables with duplicated, unsorted and far-apart levels,
levels beyond [-1, 1], magnitudes up to 65504 and +inf.
"""

import numpy as np

from oracle import bits

DYADIC_SCALES = (0x3F80, 0x3FFF, 0x3C23, 0x3A5B, 0x0001, 0x0080, 0x00FF, 0x7F7F, 0x7A01, 0x0400)


def all_finite_bf16(cols):
    """Every finite bf16 pattern (+0 .. max, then their negatives), zero-padded
    to rows of `cols`."""
    v = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)
    v = np.concatenate([v, v | 0x8000])
    pad = (-len(v)) % cols
    return np.ascontiguousarray(np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(-1, cols))


def groups_with_absmax(sb, cols):
    """Every finite bf16 value of magnitude <= sb (both signs), cols - 1 per
    row after a leading sb, so that every row's absmax is sb."""
    allpos = np.arange(0x0000, 0x7F80, dtype=np.uint32)
    vals = allpos[allpos <= sb].astype(np.uint16)
    vals = np.concatenate([vals, vals | 0x8000])
    pad = (-len(vals)) % (cols - 1)
    vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, cols - 1)
    return np.ascontiguousarray(
        np.concatenate([np.full((vals.shape[0], 1), sb, np.uint16), vals], axis=1))


def dyadic_cases():
    """(scale bits, weight [rows, 64]) for every scale of DYADIC_SCALES."""
    for sb in DYADIC_SCALES:
        yield sb, groups_with_absmax(sb, 64)


def _adversarial_tables(rows, g):
    """LUT16 tables [rows, 16] with levels far apart in magnitude, symmetric
    pairs around zero, unsorted order and entries beyond [-1, 1]."""
    kinds = []
    # tiny and unit levels mixed in random order (distances that fp32 and
    # fp64 round to the same value)
    t = bits.rne_bf16(g.choice([-1.0, 1.0], (rows, 16)) * 2.0 ** g.integers(-130, 1, (rows, 16)))
    kinds.append(t)
    # symmetric +-v pairs, every level once with each sign
    v = bits.rne_bf16(2.0 ** g.uniform(-20, 0, (rows, 8)))
    kinds.append(np.concatenate([v, v | 0x8000], axis=1))
    # unsorted levels beyond [-1, 1], including the bf16 extremes
    t = bits.rne_bf16(g.uniform(-8, 8, (rows, 16)))
    t[:, 3] = 0x7F7F
    t[:, 9] = 0xFF7F
    t[:, 11] = 0x0001
    kinds.append(t)
    return kinds


def lut16_cases():
    """(name, w [rows, 64], scales [rows, 1], tables [rows, 1, 16]) for the
    per-group codec; the LUT16S cases are the rows of lut16s_cases."""
    w = all_finite_bf16(64)
    rows = w.shape[0]
    g = np.random.default_rng(71)
    for sb in (0x3F80, 0x7F7F, 0x0001, 0x3C23):
        L = bits.rne_bf16(np.sort(g.uniform(-1, 1, (rows, 16)), axis=-1))
        L[:, 0] = 0xBF80          # -1
        L[:, 15] = 0x3F80         # +1
        L[::7, 3:5] = 0x0000      # duplicated levels
        s = np.full((rows, 1), sb, np.uint16)
        yield f"sorted s={sb:#06x}", w, s, np.ascontiguousarray(L.reshape(rows, 1, 16))
    # the uniform grid (j - 8) / 8: sorted and distinct, with every midpoint
    # (2j - 15) / 16 itself a bf16 value, so the sweep hits exact ties at all
    # of them (the lower level must win)
    grid = bits.rne_bf16((np.arange(16) - 8) / 8.0)
    for sb in (0x3F80, 0x4300):
        s = np.full((rows, 1), sb, np.uint16)
        L = np.ascontiguousarray(np.broadcast_to(grid, (rows, 1, 16)))
        yield f"grid s={sb:#06x}", w, s, L
    for i, L in enumerate(_adversarial_tables(rows, g)):
        for sb in (0x3F80, 0x0080, 0x7E00):
            s = np.full((rows, 1), sb, np.uint16)
            yield f"adversarial{i} s={sb:#06x}", w, s, np.ascontiguousarray(L.reshape(rows, 1, 16))


def lut16s_cases():
    """(name, w [rows, 64], scales [rows, 1], table [16]) for the shared-table codec."""
    w = all_finite_bf16(64)
    rows = w.shape[0]
    g = np.random.default_rng(74)
    T = bits.rne_bf16(np.sort(g.uniform(-1, 1, 16)))
    T[0], T[15] = 0xBF80, 0x3F80
    T2 = bits.rne_bf16(np.array([1e-30, -1.0, 1.0, -1e-30, 0.5, 0.25, 2.0 ** -100, -0.5,
                                 0.0, 1e-3, -1e-3, 0.75, -0.75, 2.0 ** -60, -2.0 ** -60, 0.125]))
    for sb in (0x3F80, 0x7F7F, 0x0001, 0x3C23):
        s = np.full((rows, 1), sb, np.uint16)
        yield f"T s={sb:#06x}", w, s, T
        yield f"T2 s={sb:#06x}", w, s, T2


def signmag8_cases():
    """(name, w [rows, 64], codebook [rows, 2, 8] fp16 bits)."""
    w = all_finite_bf16(64)
    ng = 2 * w.shape[0]  # groups of 32
    g = np.random.default_rng(72)
    for kind in range(6):
        if kind == 5:
            # the grid j / 8: every midpoint (2j + 1) / 16 is a bf16 value
            mags = np.broadcast_to(np.arange(8) / 8.0, (ng, 8)).copy()
        elif kind == 0:
            mags = np.sort(g.uniform(0, 0.1, (ng, 8)), axis=-1)
        elif kind == 1:
            mags = np.sort(2.0 ** g.uniform(-26, -10, (ng, 8)), axis=-1)
        elif kind == 2:
            mags = np.sort(g.uniform(0, 65504, (ng, 8)), axis=-1)
            mags[:, 7] = 65504.0
        elif kind == 3:
            # unsorted, magnitudes far apart (fp16 subnormals next to 2^15)
            mags = 2.0 ** g.integers(-24, 16, (ng, 8))
        else:
            mags = np.sort(g.uniform(0, 2, (ng, 8)), axis=-1)
        cb = bits.rne_fp16(mags)
        if kind != 5:
            cb[::5, 2] = cb[::5, 1]   # a duplicated level
            cb[::3, 0] = 0
        if kind == 4:
            cb[:, 6:] = 0x7C00    # +inf magnitudes, as the fit gives beyond fp16
            cb[::4, :] = 0x7C00   # groups whose every magnitude is +inf
        yield f"kind{kind}", w, np.ascontiguousarray(cb.reshape(w.shape[0], 2, 8))
