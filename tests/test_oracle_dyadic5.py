"""Pins for oracle/dyadic5.py (3/4/5-bit dyadic groups in one 5-bit index space).

* exact-rational brute force of the argmin for every width, with planted
  code midpoints (ties) and group extremes;
* nesting: width-4 groups give exactly twice the 4-bit codec's indices and
  the same rebuilt values (the 4-bit oracle is pinned on its own);
* |w - code| <= step / 2 for in-range weights (the top code for the rest),
  width-3 indices are multiples of 4;
* the rebuild against exact rational rounding on every 5-bit index for a
  sweep of scales, including subnormal and near-maximum ones;
* the high-bit layout is a bijection, and the two planes round-trip.
"""

import numpy as np
import pytest

import synthetic
from oracle import bits, dyadic, dyadic5
from tests import exact


def _widths(n, g, seed):
    return np.random.default_rng(seed).choice([3, 4, 5], size=(n, g)).astype(np.uint8)


def _brute(wb, sb, b):
    s = exact.bf16_fraction(sb)
    half = 2 ** (b - 1)
    if s == 0:
        return 16
    w = exact.bf16_fraction(wb)
    d = [abs(w - (s / half) * (j - half)) for j in range(2 * half)]
    return d.index(min(d)) * 2 ** (5 - b)


def test_argmin_vs_exact_rational_bruteforce():
    g = np.random.default_rng(5)
    w = synthetic.normal_bf16((4, 512), 0.02, 13)
    s = dyadic.scales(w)
    sv = bits.bf16_to_f64(s)
    widths = _widths(4, 8, 6)
    # plant exact midpoints of each group's own codebook
    for r in range(4):
        for gi in range(8):
            h = 2 ** (int(widths[r, gi]) - 1)
            for slot in (3, 17, 40):
                t = int(g.integers(0, 2 * h - 1))
                mid = (2 * t + 1 - 2 * h) / (2 * h) * sv[r, gi]
                mb = bits.rne_bf16(np.array([mid]))[0]
                if bits.bf16_to_f64(np.array([mb]))[0] == mid:
                    w[r, 64 * gi + slot] = mb
    w[0, :64] = 0
    s = dyadic.scales(w)
    idx = dyadic5.indices(w, s, widths)
    for r in range(4):
        for c in range(512):
            assert idx[r, c] == _brute(w[r, c], s[r, c // 64], int(widths[r, c // 64])), (r, c)


def test_indices_on_the_gpu_sweeps_by_midpoint_count():
    """The oracle's rule (first minimum of the fp64 distances) against a
    different route to the nearest code, on the inputs of the GPU's
    exhaustive DYADIC5 test (every finite bf16 value of magnitude <= s, seven
    scales, widths 3 / 4 / 5): the codes are sorted and distinct, so the
    lowest nearest one is the number of midpoints strictly below w; each
    midpoint s (2t + 1 - 2h) / (2h) is exact in double, and so is each
    comparison with a bf16 weight."""
    from tests import sweeps
    for sb in (0x3F80, 0x3FFF, 0x3C23, 0x0001, 0x0080, 0x7F7F, 0x7A01):
        w = sweeps.groups_with_absmax(sb, 64)
        widths = np.resize(np.array([3, 4, 5], np.uint8), (w.shape[0], 1))
        s = dyadic.scales(w)
        got = dyadic5.indices(w, s, widths)
        wv = bits.bf16_to_f64(w)
        sv = bits.bf16_to_f64(s)[:, 0]
        for r in range(w.shape[0]):
            h = 2 ** (int(widths[r, 0]) - 1)
            if sv[r] == 0.0:
                want = np.full(64, 16, np.uint8)
            else:
                mids = sv[r] * (2 * np.arange(2 * h - 1) + 1 - 2 * h) / (2 * h)
                j = (wv[r][:, None] > mids[None, :]).sum(axis=1)
                want = (j * 2 ** (5 - int(widths[r, 0]))).astype(np.uint8)
            assert np.array_equal(got[r], want), (hex(sb), r)


def test_width4_nests_in_the_4bit_codec():
    w = synthetic.student_t_bf16((16, 1024), 4, 0.02, 17)
    w[3, 64:128] = 0
    s = dyadic.scales(w)
    idx4 = dyadic.indices(w, s)
    idx5 = dyadic5.indices(w, s, np.full((16, 16), 4, np.uint8))
    assert np.array_equal(idx5, 2 * idx4.astype(np.uint8))
    assert np.array_equal(dyadic5.dequant_from_indices(idx5, s), dyadic.dequant_from_indices(idx4, s))


def test_error_bound_and_grid():
    w = synthetic.normal_bf16((8, 1024), 0.02, 19)
    widths = _widths(8, 16, 20)
    idx, s = dyadic5.quantize(w, widths)
    assert np.all(idx[widths.repeat(64, axis=1) == 3] % 4 == 0)
    assert np.all(idx[widths.repeat(64, axis=1) == 4] % 2 == 0)
    sv = bits.bf16_to_f64(s).repeat(64, axis=1)
    half = 2.0 ** (widths.repeat(64, axis=1).astype(np.int64) - 1)
    step = sv / half
    code = sv / 16.0 * (idx.astype(np.float64) - 16.0)
    wv = bits.bf16_to_f64(w)
    # in range: up to half a step above the top code (half - 1) * step
    inr = wv <= (half - 0.5) * step
    assert np.all(np.abs(wv - code)[inr] <= step[inr] / 2)
    # above it (only +absmax-like weights): the top code
    assert np.all(code[~inr] == ((half - 1) * step)[~inr])


def _rne_int(sbits, j5):
    """Exact rebuild: an exact zero product is +0; a nonzero product that
    rounds to zero keeps its sign."""
    v = exact.bf16_fraction(sbits) / 16 * (j5 - 16)
    if v == 0:
        return 0
    r = exact.rne_bf16_fraction(v)
    if r == 0:
        return 0x8000 if v < 0 else 0
    return exact.fraction_to_bf16_bits(r)


@pytest.mark.parametrize("sbits", [0x3C23, 0x0001, 0x007F, 0x0080, 0x1234, 0x7F7F, 0x7E01, 0x4F00])
def test_dequant_every_index_vs_exact(sbits):
    idx = np.tile(np.arange(32, dtype=np.uint8), 2)[None, :]
    out = dyadic5.dequant_from_indices(idx, np.array([[sbits]], np.uint16))
    for j in range(64):
        assert out[0, j] == _rne_int(sbits, j % 32), (hex(sbits), j)


def _rne_int_fast(sbits, j5):
    """RNE_bf16((s/16)(j5 - 16)) in integer arithmetic (the same result as
    _rne_int, fast enough for every scale): an exact zero is +0, a nonzero
    product rounding to zero keeps its sign."""
    d = j5 - 16
    e, m = (sbits >> 7) & 0xFF, sbits & 0x7F
    S, a = (m, -133) if e == 0 else (m + 128, e - 134)    # |s| = S * 2**a
    if S == 0 or d == 0:
        return 0
    sign = 0x8000 if (d < 0) != (sbits >= 0x8000) else 0
    P, f = S * abs(d), a - 4                                # |value| = P * 2**f
    q = max(P.bit_length() - 1 + f - 7, -133)
    sh = q - f
    if sh <= 0:
        r = P << (-sh)
    else:
        r, rem = P >> sh, P & ((1 << sh) - 1)
        if rem > (1 << (sh - 1)) or (rem == (1 << (sh - 1)) and r & 1):
            r += 1
    if r == 256:
        r, q = 128, q + 1
    if r < 128:
        return sign | r                                     # subnormal, or rounded to zero
    return sign | ((q + 134) << 7) | (r - 128)


def test_dequant_every_scale_every_index():
    """Every finite bf16 scale of either sign x all 32 indices against the
    integer rounding, which agrees with the exact-fraction rounding above on
    the scales that test uses."""
    for sb in (0x3C23, 0x0001, 0x007F, 0x0080, 0x1234, 0x7F7F, 0x7E01, 0x4F00, 0xBC23, 0x8001):
        for j in range(32):
            assert _rne_int_fast(int(sb), j) == _rne_int(int(sb), j), (hex(sb), j)
    allb = bits.all_finite_bf16()
    idx = np.tile(np.arange(32, dtype=np.uint8), 2)[None, :].repeat(len(allb), axis=0)
    got = dyadic5.dequant_from_indices(idx, allb[:, None])[:, :32]
    want = np.array([[_rne_int_fast(int(sb), j) for j in range(32)] for sb in allb], np.uint16)
    assert np.array_equal(got, want)


def test_msb_layout_is_a_bijection():
    pos = sorted(dyadic5.msb_bit(i) for i in range(32))
    assert pos == list(range(32))


def test_planes_roundtrip():
    g = np.random.default_rng(23)
    idx = g.integers(0, 32, size=(5, 256)).astype(np.uint8)
    nib, msb = dyadic5.planes(idx)
    assert nib.shape == (5, 128) and msb.shape == (5, 32)
    assert np.array_equal(dyadic5.unplanes(nib, msb), idx)
    # a single high bit lands where the layout says
    one = np.zeros((1, 32), np.uint8)
    one[0, 13] = 16
    _, m = dyadic5.planes(one)
    assert int(m.view("<u4")[0, 0]) == 1 << dyadic5.msb_bit(13)
