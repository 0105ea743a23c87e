"""Pins for oracle/lut16.py and oracle/signmag8.py (and the shared Lloyd fit).

The nearest-level decision, dequant and fit of both LUT codecs are pinned by
exact-rational brute force, exact special cases, the Lloyd monotonicity the
int4-g32 page states (section 1.3: the per-weight MSE never rises from one
round to the next), the optimal 1D k-means cost computed by dynamic
programming, and agreement between the numpy and C implementations.
"""

from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle import bits, lut16, native, packing, signmag8
from tests import exact


def _lut_data(rows=8, k=512, seed=21):
    return synthetic.normal_outliers_bf16((rows, k), 0.015, 0.001, 0.15, seed)


# ------------------------------------------------------------------ LUT16 argmin
def test_lut16_decision_vs_exact_argmin():
    w = _lut_data()
    s, L = lut16.fit(w)
    idx = lut16.indices(w, s, L)
    n, k = w.shape
    mism = 0
    for r in range(n):
        for c in range(0, k, 3):
            g = c // 64
            sv = exact.bf16_fraction(s[r, g])
            lv = [sv * exact.bf16_fraction(x) for x in L[r, g]]
            wv = exact.bf16_fraction(w[r, c])
            d = [abs(wv - v) for v in lv]
            want = d.index(min(d))
            mism += int(idx[r, c] != want)
    assert mism == 0


def test_lut16_decision_ties_go_low_and_fp32_rule():
    # two equal levels -> lower index; an exact midpoint -> lower index
    s = np.array([[0x3F80]], np.uint16)                     # s = 1
    L = np.zeros((1, 1, 16), np.uint16)
    L[0, 0, :] = bits.rne_bf16(np.linspace(-1, 1, 16))
    L[0, 0, 9] = L[0, 0, 4]                                  # duplicate level
    w = np.zeros((1, 64), np.uint16)
    lv = bits.bf16_to_f64(L[0, 0])
    w[0, 0] = L[0, 0, 4]
    mid = (lv[10] + lv[11]) / 2
    w[0, 1] = bits.rne_bf16(np.array([mid]))[0]
    idx = lut16.indices(w, s, L)
    assert idx[0, 0] == 4
    wv = bits.bf16_to_f64(w[0, 1:2])[0]
    d = np.abs(wv - lv)
    assert idx[0, 1] == int(np.flatnonzero(d == d.min())[0])


def test_lut16_dequant_exact_product_rounding():
    w = _lut_data(4, 256, 22)
    s, L = lut16.fit(w)
    p = lut16.quantize_pack(w, s, L)
    deq = lut16.dequant(p, s, L)
    idx = packing.unpack(p)
    for r in range(4):
        for c in range(0, 256, 5):
            v = exact.bf16_fraction(s[r, c // 64]) * exact.bf16_fraction(L[r, c // 64, idx[r, c]])
            assert deq[r, c] == exact.fraction_to_bf16_bits(exact.rne_bf16_fraction(v)) or (
                v == 0 and deq[r, c] in (0, 0x8000))


def _rne_bf16_product_int(abits, bbits):
    """Bits of RNE_bf16(a * b) for two finite bf16 numbers, in integer
    arithmetic (overflow to +-inf, a zero result keeps the product's sign)."""
    def dec(u):
        e, m = (u >> 7) & 0xFF, u & 0x7F
        return (m, -133) if e == 0 else (m + 128, e - 134)   # value = S * 2**a
    abits, bbits = int(abits), int(bbits)
    sign = 0x8000 if (abits ^ bbits) & 0x8000 else 0
    (sa, ea), (sb, eb) = dec(abits), dec(bbits)
    P, f = sa * sb, ea + eb
    if P == 0:
        return sign
    q = max(P.bit_length() - 1 + f - 7, -133)   # exponent of the result's last bit
    sh = q - f
    if sh <= 0:
        r = P << (-sh)
    else:
        r, rem = P >> sh, P & ((1 << sh) - 1)
        half = 1 << (sh - 1)
        if rem > half or (rem == half and r & 1):
            r += 1
    if r == 256:
        r, q = 128, q + 1
    if r < 128:
        return sign | r                           # subnormal or zero
    E = q + 134
    if E >= 255:
        return sign | 0x7F80
    return sign | (E << 7) | (r - 128)


def test_lut16_dequant_every_level_extreme_scales():
    """RNE_bf16(s * L) for every finite bf16 level (tables beyond [-1, 1],
    signed zeros, subnormals) under scales from the smallest subnormal to the
    largest finite bf16 (both signs), against integer rounding: the products
    overflow, round to the largest finite value, or underflow.  The scales
    include every one the GPU's extreme-table dequant test uses."""
    allb = bits.all_finite_bf16()
    scales = np.array([0x0001, 0x0080, 0x3F80, 0x7F7F, 0x7F00, 0x4000, 0x00FF, 0x3C23,
                       0xBF80, 0x8001], np.uint16)
    n = (len(allb) + 15) // 16
    levels = np.resize(allb, n * 16).reshape(n, 1, 16)
    idx = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :].repeat(n, axis=0)
    for sb in scales:
        s = np.full((n, 1), sb, np.uint16)
        want = np.array([[_rne_bf16_product_int(sb, l) for l in row] for row in levels[:, 0]],
                        np.uint16)
        got = lut16.dequant_from_indices(idx, s, levels)[:, :16]
        assert np.array_equal(got, want), hex(sb)


# ------------------------------------------------------------------ Lloyd
def _optimal_kmeans_cost(x, k):
    """Optimal 1D k-means SSE by dynamic programming over the sorted points
    (segment costs computed directly, no prefix-sum cancellation)."""
    x = np.sort(np.asarray(x, dtype=np.float64))
    n = len(x)
    cost = np.full((n + 1, n + 1), np.inf)
    for i in range(n):
        for j in range(i + 1, n + 1):
            seg = x[i:j]
            cost[i, j] = np.sum((seg - seg.mean()) ** 2)
    dp = np.full((k + 1, n + 1), np.inf)
    dp[0, 0] = 0.0
    for c in range(1, k + 1):
        for j in range(c, n + 1):
            dp[c, j] = np.min(dp[c - 1, c - 1:j] + cost[c - 1:j, j])
    return float(np.min(dp[1:, n]))


def test_lloyd_monotone_and_above_optimum():
    g = np.random.default_rng(5)
    u = g.standard_t(4, (40, 64)) / 6
    c0 = lut16.quantile_init(u, 16)
    c, hist = lut16.lloyd(u, c0, 25, history=True)
    assert np.all(np.diff(hist, axis=-1) <= 1e-15)
    for r in range(0, 40, 8):
        opt = _optimal_kmeans_cost(list(u[r]), 16) / 64
        assert hist[r, -1] >= opt * (1 - 1e-12)


def test_lloyd_separated_clusters_reach_exact_means():
    g = np.random.default_rng(6)
    centres = np.arange(16) * 10.0
    pts = (centres[:, None] + g.integers(-2, 3, (16, 4))).astype(np.float64)
    u = g.permutation(pts.ravel())[None, :]
    c = lut16.lloyd(u, lut16.quantile_init(u, 16), 25)[0]
    for q in range(16):
        mem = [Fraction(int(v)) for v in pts[q]]
        assert Fraction(c[q]) == sum(mem) / 4


def test_lloyd_known_fixed_point_two_clusters():
    # points {0,1,2,10}: quantile start (k=2, stride 2) -> c = {1, 10};
    # assignment {0,1,2}|{10} gives means {1, 10}: a fixed point.
    u = np.array([[10.0, 0.0, 2.0, 1.0]])
    c = lut16.lloyd(u, lut16.quantile_init(u, 2), 25)
    assert list(c[0]) == [1.0, 10.0]
    # points {0, 4, 5, 6}: start {4, 6}; round 1: {0,4}|{5,6} -> {2, 5.5};
    # round 2: {0}|{4,5,6} -> {0, 5}; then stable.
    u = np.array([[0.0, 4.0, 5.0, 6.0]])
    c, h = lut16.lloyd(u, lut16.quantile_init(u, 2), 25, history=True)
    assert list(c[0]) == [0.0, 5.0]


def test_lut16_fit_recovers_16_point_groups():
    # a group of 16 distinct values, each 4 times, with absmax 1: exact recovery
    g = np.random.default_rng(7)
    vals = np.sort(g.choice(np.arange(-127, 128), 16, replace=False)) / 128.0
    vals[-1] = 1.0
    w = bits.rne_bf16(g.permutation(np.repeat(vals, 4)))[None, :]
    s, L = lut16.fit(w)
    assert np.array_equal(bits.bf16_to_f64(L[0, 0]), vals)
    p = lut16.quantize_pack(w, s, L)
    assert np.array_equal(lut16.dequant(p, s, L), w)


def test_lut16_zero_group():
    w = np.zeros((1, 64), np.uint16)
    s, L = lut16.fit(w)
    assert s[0, 0] == 0 and np.all(L == 0)
    p = lut16.quantize_pack(w, s, L)
    assert np.all(lut16.dequant(p, s, L) == 0)


def test_lut16_c_matches_python():
    w = _lut_data(16, 1024, 23)
    w[2, :64] = 0
    s, L = lut16.fit(w)
    s2, L2 = native.lut16_fit(w)
    assert np.array_equal(s, s2) and np.array_equal(L, L2)
    assert np.array_equal(lut16.indices(w, s, L), native.lut16_indices(w, s, L))


def tie_groups():
    """bf16 groups whose fit depends on tie rules: runs of -0.0 / +0.0 in both
    orders (the quantile start lands on zeros, some centres stay empty), few
    distinct values, repeated values, an all-zero group, tiny and huge
    magnitudes.  Shared with the GPU parity test of the fit."""
    g = np.random.default_rng(29)
    rows = []
    z = np.zeros(64, np.uint16)
    a = z.copy(); a[0:40:2] = 0x8000; a[40:] = bits.rne_bf16(np.arange(1, 25) / 24.0)
    rows.append(a)
    b = z.copy(); b[1:40:2] = 0x8000; b[40:] = bits.rne_bf16(-np.arange(1, 25) / 24.0)
    rows.append(b)
    c = bits.rne_bf16(g.choice([-0.5, 0.25, 1.0], 64))       # three distinct values
    rows.append(c)
    d = bits.rne_bf16(np.repeat(g.normal(0, 0.02, 8), 8))   # eight values, 8 times each
    rows.append(d)
    rows.append(z.copy())                                    # all zero
    e = (g.integers(0x0001, 0x0080, 64) | (g.integers(0, 2, 64) << 15)).astype(np.uint16)
    rows.append(e)                                           # subnormal bf16 only
    f = (g.integers(0x7E00, 0x7F7F, 64) | (g.integers(0, 2, 64) << 15)).astype(np.uint16)
    rows.append(f)                                           # magnitudes near the bf16 max
    h = z.copy(); h[5] = 0x3F80; h[9] = 0x8000               # one nonzero value
    rows.append(h)
    return np.stack(rows).reshape(2, 4 * 64)


def test_lut16_c_matches_python_on_ties():
    w = tie_groups()
    for iters in (0, 1, 25):
        s, L = lut16.fit(w, iters)
        s2, L2 = native.lut16_fit(w, iters)
        assert np.array_equal(s, s2) and np.array_equal(L, L2), iters
    # the quantile start on zero runs keeps the zeros' signs in element order
    s0, L0 = lut16.fit(w, 0)
    u = bits.bf16_to_f64(w[0, :64])
    order = sorted(range(64), key=lambda i: (u[i], i))   # stable by element index
    want = np.array([w[0, order[4 * q + 2]] for q in range(16)], np.uint16)
    assert np.array_equal(L0[0, 0], bits.rne_bf16(bits.bf16_to_f64(want)))


# ------------------------------------------------------------------ LUT16S
def test_lut16s_fit_equals_group_fit_on_one_group():
    # with a single group the whole-weight fit and the per-group fit coincide
    for seed in (1, 2, 3):
        w = synthetic.normal_outliers_bf16((1, 64), 0.015, 0.05, 0.15, seed)
        s, L = lut16.fit(w)
        s2, T = lut16.fit_shared(w)
        assert np.array_equal(s, s2) and np.array_equal(L[0, 0], T)


def test_lut16s_fit_recovers_16_values_and_roundtrips():
    # every group holds the same 16 normalised values (4 copies each, absmax 1)
    # times a power-of-two scale: the start already sits on them, Lloyd keeps
    # them, and quantize -> dequant reproduces the weight exactly
    g = np.random.default_rng(11)
    vals = np.sort(g.choice(np.arange(-127, 128), 16, replace=False)) / 128.0
    vals[-1] = 1.0
    rows = []
    for r in range(6):
        groups = [g.permutation(np.repeat(vals, 4)) * 2.0 ** int(g.integers(-20, 5))
                  for _ in range(3)]
        rows.append(np.concatenate(groups))
    w = bits.rne_bf16(np.stack(rows))
    s, T = lut16.fit_shared(w)
    assert np.array_equal(bits.bf16_to_f64(T), vals)
    tables = lut16.shared_tables(s, T)
    p = lut16.quantize_pack(w, s, tables)
    assert np.array_equal(lut16.dequant(p, s, tables), w)
    assert np.array_equal(s, lut16.group_scales(w))


def test_lut16s_zero_groups_and_scale():
    w = _lut_data(4, 256, 41)
    w[1, 64:128] = 0
    s, T = lut16.fit_shared(w)
    assert s[1, 1] == 0
    tables = lut16.shared_tables(s, T)
    d = lut16.dequant(lut16.quantize_pack(w, s, tables), s, tables)
    assert np.all(bits.bf16_to_f64(d[1, 64:128]) == 0)


# ------------------------------------------------------------------ SIGNMAG8
def _sm_data(rows=8, k=512, seed=31):
    return synthetic.student_t_bf16((rows, k), 5, 0.02, seed)


def test_signmag8_decision_vs_exact():
    w = _sm_data()
    cb = signmag8.fit(w)
    nib = signmag8.indices(w, cb)
    for r in range(8):
        for c in range(0, 512, 3):
            g = c // 32
            wv = exact.bf16_fraction(w[r, c])
            m = [exact.f16_fraction(x) for x in cb[r, g]]
            d = [abs(abs(wv) - v) for v in m]
            want = d.index(min(d)) | (8 if wv < 0 else 0)
            assert nib[r, c] == want


def test_signmag8_dequant_sign_and_exact_levels():
    w = _sm_data(4, 256, 32)
    w[0, 0] = 0x8000        # -0.0 -> sign bit 0
    cb = signmag8.fit(w)
    cb[1, 0, 0] = 0         # a zero magnitude level
    p = signmag8.quantize_pack(w, cb)
    nib = packing.unpack(p)
    assert nib[0, 0] >> 3 == 0
    deq = signmag8.dequant(p, cb)
    for r in range(4):
        for c in range(256):
            mag = exact.f16_fraction(cb[r, c // 32, nib[r, c] & 7])
            neg = bool(nib[r, c] & 8)
            assert exact.f16_fraction(deq[r, c]) == (-mag if neg else mag)
            assert bool(deq[r, c] & 0x8000) == neg        # -0.0 reproduced
    # the sign bit is exactly w < 0
    wv = bits.bf16_to_f64(w)
    assert np.array_equal((nib >> 3).astype(bool), wv < 0)


def test_signmag8_dequant_every_magnitude():
    """(nib & 8 ? -1 : +1) * M for every finite fp16 magnitude pattern (both
    zeros, subnormals, the largest) and +-inf, with both signs, as exact values:
    the oracle's rebuild is the exact product by +-1."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    pats = u[((u >> 10) & 0x1F) != 0x1F]                        # every finite fp16
    pats = np.concatenate([pats, np.array([0x7C00, 0xFC00], np.uint16)])
    n = (len(pats) + 7) // 8
    cb = np.resize(pats, n * 8).reshape(n, 1, 8)
    nib = np.tile(np.arange(16, dtype=np.uint8), 2)[None, :].repeat(n, axis=0)   # [n, 32]
    deq = signmag8.dequant_from_indices(nib, cb)
    for r in range(n):
        for c in range(16):
            m = int(cb[r, 0, c & 7])
            got = int(deq[r, c])
            if (m & 0x7FFF) == 0x7C00:                           # +-inf
                assert got & 0x7FFF == 0x7C00
                assert bool(got & 0x8000) == (bool(m & 0x8000) != bool(c & 8))
                continue
            want = exact.f16_fraction(m) * (-1 if c & 8 else 1)
            assert exact.f16_fraction(got) == want, (hex(m), c)
            if want == 0:                                        # the sign of a zero product
                assert bool(got & 0x8000) == (bool(m & 0x8000) != bool(c & 8))


def test_signmag8_fit_monotone_and_c_matches():
    w = _sm_data(16, 1024, 33)
    cb = signmag8.fit(w)
    assert np.array_equal(cb, native.signmag8_fit(w))
    assert np.array_equal(signmag8.indices(w, cb), native.signmag8_indices(w, cb))
    a = np.abs(bits.bf16_to_f64(w)).reshape(-1, 32)
    _, h = lut16.lloyd(a, lut16.quantile_init(a, 8), 25, history=True)
    assert np.all(np.diff(h, axis=-1) <= 1e-15)


def signmag8_tie_groups():
    """bf16 groups of 32 whose SIGNMAG8 fit depends on ties and on the fp16
    rounding: +-x pairs (equal magnitudes), signed zeros, few distinct
    magnitudes, magnitudes whose centres round to fp16 subnormals, to zero,
    to the fp16 maximum or overflow to infinity.  Shared with the GPU parity
    test of the fit."""
    g = np.random.default_rng(31)
    rows = []
    z = np.zeros(32, np.uint16)
    a = bits.rne_bf16(np.repeat(g.normal(0, 0.02, 16), 2) * np.tile([1, -1], 16))
    rows.append(a)                                           # +-x pairs
    b = z.copy(); b[0:20:2] = 0x8000; b[20:] = bits.rne_bf16(-np.arange(1, 13) / 12.0)
    rows.append(b)                                           # signed zeros + a ramp
    rows.append(bits.rne_bf16(g.choice([-0.5, 0.25, 1.0, -1.0], 32)))
    rows.append(z.copy())                                    # all zero
    # magnitudes between 2^-27 and 2^-13: fp16 subnormals, zero and the first normals
    rows.append(bits.rne_bf16(g.choice([-1, 1], 32) * 2.0 ** g.uniform(-27, -13, 32)))
    # magnitudes around the fp16 maximum 65504 and the overflow threshold 65520
    rows.append(bits.rne_bf16(g.choice([-1, 1], 32) * g.uniform(64000, 67000, 32)))
    rows.append((g.integers(0x7E00, 0x7F7F, 32) | (g.integers(0, 2, 32) << 15)).astype(np.uint16))
    h = z.copy(); h[7] = 0xBF80
    rows.append(h)                                           # one nonzero value
    return np.stack(rows).reshape(2, 4 * 32)


def test_signmag8_c_matches_python_on_ties():
    w = signmag8_tie_groups()
    for iters in (0, 1, 25):
        cb = signmag8.fit(w, iters)
        assert np.array_equal(cb, native.signmag8_fit(w, iters)), iters
    cb = signmag8.fit(w, 25)
    # the overflow and subnormal cases are reached
    assert np.any(cb == 0x7C00) and np.any((cb > 0) & (cb < 0x0400))
    # 0 rounds: the centres are the magnitudes of sorted rank 4q + 2
    a = np.sort(np.abs(bits.bf16_to_f64(w[0, :32])))
    assert np.array_equal(signmag8.fit(w, 0)[0, 0], bits.rne_fp16(a[2::4]))


# ------------------------------------------------------------------ LUT16S_IL layout
def test_interleave_layout_by_hand():
    """One row of k = 512: two records of 144 bytes, each the block's 128
    packed bytes, its four scales little-endian, then 8 zero bytes."""
    packed = (np.arange(256) % 251).astype(np.uint8)[None, :]
    scales = np.array([[0x1234, 0xABCD, 0x0001, 0xFF00, 0x0102, 0x0304, 0x0506, 0x0708]], np.uint16)
    il = lut16.interleave(packed, scales)
    assert il.shape == (1, 288)
    assert list(il[0, :128]) == list(packed[0, :128])
    assert list(il[0, 128:144]) == [0x34, 0x12, 0xCD, 0xAB, 0x01, 0x00, 0x00, 0xFF] + [0] * 8
    assert list(il[0, 144:272]) == list(packed[0, 128:])
    assert list(il[0, 272:288]) == [0x02, 0x01, 0x04, 0x03, 0x06, 0x05, 0x08, 0x07] + [0] * 8


def test_interleave_roundtrip():
    g = np.random.default_rng(12)
    packed = g.integers(0, 256, (7, 1024)).astype(np.uint8)     # k = 2048
    scales = g.integers(0, 1 << 16, (7, 32)).astype(np.uint16)
    p2, s2 = lut16.deinterleave(lut16.interleave(packed, scales))
    assert np.array_equal(p2, packed) and np.array_equal(s2, scales)
