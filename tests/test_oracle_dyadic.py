"""Pins for oracle/dyadic.py and oracle/packing.py.

What fixes the dyadic codec without any implementation to compare against:
the page's printed codebook (golden fixture), exact-rational brute force on
small inputs, an exhaustive sweep against the textbook symmetric INT4
round-to-nearest written in integer arithmetic, the codec's invariants, and
an exhaustive dequant sweep against integer rounding.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import synthetic
from oracle import bits, dyadic, native, packing
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------ golden
def test_codebook_matches_page():
    rows = _read_table("dyadic_codebook_b4.txt")
    c = dyadic.codebook(np.array([1.0]))[0]
    assert len(rows) == 16
    for j, (i, v) in enumerate(rows):
        assert int(i) == j and c[j] == float(v)


def test_int4_range_matches_survey_page():
    rows = dict(_read_table("int4_range.txt"))
    c = dyadic.codebook(np.array([8.0]))[0]     # step 1 -> integer codes
    assert c.min() == float(rows["qmin"]) and c.max() == float(rows["qmax"])


def test_packing_examples():
    for lo, hi, byte in _read_table("packing_examples.txt"):
        p = packing.pack(np.array([[int(lo), int(hi)]], dtype=np.uint8))
        assert p[0, 0] == int(byte, 16)
        assert list(packing.unpack(p)[0]) == [int(lo), int(hi)]


def test_pack_roundtrip_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(2, 128)
    assert np.array_equal(packing.pack(packing.unpack(b)), b)
    g = np.random.default_rng(0)
    idx = g.integers(0, 16, (7, 64)).astype(np.uint8)
    assert np.array_equal(packing.unpack(packing.pack(idx)), idx)


def test_storage_accounting_matches_pages():
    t = {k: float(v) for k, v in _read_table("storage_accounting.txt")}
    n = int(t["dg_weights"])
    packed = n // 2
    scales = packing.storage_bytes(n, 64, 2) - packed
    assert round(packed / 1e6) == t["dg_packed_mb"]
    assert round(scales / 1e6) == t["dg_scale_mb"]
    assert round(packing.storage_bytes(n, 64, 2) / 1e6) == t["dg_total_mb"]
    assert round(t["dg_bf16_mb"] / t["dg_total_mb"]) == t["dg_ratio"]
    # int4-g32 page: 4 bits per weight plus 8 parameter bits per group of 32
    bpw = 4 + 8 / 32
    assert bpw == t["g32_bits_per_weight"] and round(16 / bpw, 2) == t["g32_ratio"]


# ------------------------------------------------------------------ scale
def test_scale_is_group_absmax_along_k():
    g = np.random.default_rng(1)
    w = bits.rne_bf16(g.standard_normal((3, 192)))
    s = dyadic.scales(w)
    for r in range(3):
        for gi in range(3):
            m = max(abs(exact.bf16_fraction(x)) for x in w[r, 64 * gi:64 * gi + 64])
            assert exact.bf16_fraction(s[r, gi]) == m


# ------------------------------------------------------------------ argmin
def _brute_exact(wb, sb):
    s = exact.bf16_fraction(sb)
    if s == 0:
        return 8
    w = exact.bf16_fraction(wb)
    d = [abs(w - (s / 8) * (j - 8)) for j in range(16)]
    return d.index(min(d))


def test_argmin_vs_exact_rational_bruteforce():
    g = np.random.default_rng(2)
    w = synthetic.normal_bf16((4, 512), 0.02, 11)
    # plant exact midpoints and group extremes
    s = dyadic.scales(w)
    sv = bits.bf16_to_f64(s)
    for r in range(4):
        for gi in range(8):
            t = g.integers(0, 15)
            mid = (2 * t - 15) / 16 * sv[r, gi]
            mb = bits.rne_bf16(np.array([mid]))[0]
            if bits.bf16_to_f64(np.array([mb]))[0] == mid and abs(mid) <= sv[r, gi]:
                w[r, 64 * gi + 5] = mb
    s = dyadic.scales(w)
    idx = dyadic.indices(w, s)
    for r in range(4):
        for c in range(512):
            assert idx[r, c] == _brute_exact(w[r, c], s[r, c // 64]), (r, c)


def _rtn_int(wbits, sbits):
    """Symmetric INT4 round-to-nearest with ties toward the lower level, in
    exact integer arithmetic: idx = #{t in 0..14 : 16*w > (2t-15)*s}."""
    W, a = exact.bf16_int_parts(wbits)
    S, b = exact.bf16_int_parts(np.full_like(np.asarray(wbits), sbits))
    out = np.zeros(W.shape, dtype=np.int64)
    tiny = a < b - 40          # |w| < s * 2**-32: strictly inside the zero bin
    c = np.minimum(a, b)
    lhs = W * (2 ** np.minimum(a - c + 4, 62))    # 16*w in units of 2**c
    for t in range(15):
        rhs = (2 * t - 15) * S * (2 ** np.minimum(b - c, 62))
        out += (lhs > rhs).astype(np.int64)
    return np.where(tiny, 8, out)


@pytest.mark.parametrize("sbits", [0x3F80, 0x3F81, 0x3FFF, 0x3D23, 0x0001, 0x007F, 0x0080,
                                   0x0301, 0x7F7F, 0x7F00, 0x4B80, 0x1234])
def test_argmin_exhaustive_vs_int4_rtn(sbits):
    """Every finite bf16 w with |w| <= s against the textbook INT4 rounding."""
    allb = bits.all_finite_bf16()
    s = bits.bf16_to_f64(np.array([sbits], np.uint16))[0]
    w = allb[np.abs(bits.bf16_to_f64(allb)) <= s]
    # make the group's absmax equal to s: put w's in groups of 63 plus s itself
    pad = (-len(w)) % 63
    w = np.concatenate([w, np.zeros(pad, np.uint16)]).reshape(-1, 63)
    grp = np.concatenate([w, np.full((w.shape[0], 1), sbits, np.uint16)], axis=1)
    grp = grp.reshape(1, -1)
    sc = dyadic.scales(grp)
    assert np.all(sc == sbits)
    idx = dyadic.indices(grp, sc).reshape(-1, 64)[:, :63].ravel()
    want = _rtn_int(w.ravel(), sbits)
    assert np.array_equal(idx.astype(np.int64), want)


def test_argmin_invariants():
    w = synthetic.normal_bf16((64, 1024), 0.02, 12)
    s = dyadic.scales(w)
    idx = dyadic.indices(w, s).astype(np.int64)
    wv = bits.bf16_to_f64(w).reshape(64, 16, 64)
    sv = bits.bf16_to_f64(s)[..., None]
    step = sv / 8
    iv = idx.reshape(64, 16, 64)
    code = step * (iv - 8)
    assert np.all(iv[wv == 0] == 8)
    assert np.all(iv[wv == -sv.repeat(64, -1)] == 0)
    assert np.all(iv[wv == sv.repeat(64, -1)] == 15)
    inr = wv <= 7.5 * step
    assert np.all(np.abs(wv - code)[inr] <= step.repeat(64, -1)[inr] / 2)
    # monotone non-decreasing in w inside a group
    o = np.argsort(wv, axis=-1, kind="stable")
    assert np.all(np.diff(np.take_along_axis(iv, o, -1), axis=-1) >= 0)


def test_all_zero_group():
    w = np.zeros((2, 128), np.uint16)
    w[1, 70] = 0x3C00
    p, s = dyadic.quantize_pack(w)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(packing.unpack(p)[0] == 8) and np.all(packing.unpack(p)[1, :64] == 8)
    deq = dyadic.dequant(p, s)
    assert np.all(deq[0] == 0) and np.all(deq[1, :64] == 0)   # +0.0 bit patterns


# ------------------------------------------------------------------ dequant
def _dequant_int(sbits, idx):
    """RNE_bf16((s/8)*(idx-8)) in integer arithmetic, zero -> +0."""
    sbits = int(sbits)
    e = (sbits >> 7) & 0xFF
    m = sbits & 0x7F
    S, a = (m, -133) if e == 0 else (m + 128, e - 134)
    d = idx - 8
    if S == 0 or d == 0:
        return 0
    P = S * abs(d)
    f = a - 3                       # value = P * 2**f
    top = P.bit_length() - 1 + f
    q = max(top - 7, -133)
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
        assert q == -133
        out = r
    else:
        out = ((q + 7 + 127) << 7) | (r - 128)
        assert q + 7 + 127 < 255
    return out | (0x8000 if (d < 0) != (sbits >= 0x8000) else 0)


def test_dequant_exhaustive_all_scales():
    """Every finite bf16 scale of either sign (a caller may pass its own
    scales) x every index, numpy and C oracles, against the integer RNE."""
    allb = bits.all_finite_bf16()
    idx = np.arange(16, dtype=np.uint8)
    # one "row" per scale: 64 copies of the 16 indices with the scale repeated
    rows = np.tile(idx, (len(allb), 4))
    want = np.array([[_dequant_int(s, j) for j in range(16)] for s in allb], dtype=np.uint16)
    assert np.array_equal(dyadic.dequant_from_indices(rows, allb[:, None])[:, :16], want)
    assert np.array_equal(native.dyadic_dequant(rows, allb[:, None])[:, :16], want)


def test_dequant_on_code_grid():
    w = synthetic.normal_bf16((16, 512), 0.02, 13)
    p, s = dyadic.quantize_pack(w)
    deq = dyadic.dequant(p, s)
    idx = packing.unpack(p)
    for r in range(0, 16, 5):
        for c in range(0, 512, 7):
            code = exact.bf16_fraction(s[r, c // 64]) / 8 * (int(idx[r, c]) - 8)
            want = exact.fraction_to_bf16_bits(exact.rne_bf16_fraction(code))
            assert deq[r, c] == want


# ------------------------------------------------------------------ C oracle
def test_c_oracle_matches_python():
    w = synthetic.normal_bf16((32, 1024), 0.02, 14)
    w[3, :64] = 0
    w[4, 64:128] = 0x0001          # subnormal group
    w[5, 128] = 0x7F7F             # huge absmax
    idx_c, s_c = native.dyadic_quantize(w)
    p, s = dyadic.quantize_pack(w)
    assert np.array_equal(s, s_c) and np.array_equal(packing.unpack(p), idx_c)
    assert np.array_equal(dyadic.dequant(p, s), native.dyadic_dequant(idx_c, s_c))
