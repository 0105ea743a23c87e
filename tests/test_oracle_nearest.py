"""Pins for the exact nearest-level rule of the LUT16, LUT16S and SIGNMAG8
codecs (oracle/nearest.py, used by oracle/lut16.py and oracle/signmag8.py)
and for the C oracle that the GPU parity tests check against.

The rule (k-means page, section 1.2: the nearest centre; int4-g32 page,
section 1.3 step 4: the nearest level) is read as the lowest index at the
smallest exact distance.  The pin is a brute force on Python integers (every
bf16 value times 2**133, every product of two bf16 values times 2**266, is an
integer), over every finite bf16 weight, with the same scales, tables and
codebooks the GPU sweeps use (tests/sweeps.py).
"""

import numpy as np
import pytest

from oracle import bits, dyadic, lut16, native, signmag8
from tests import exact, sweeps


N_LUT16 = sum(1 for _ in sweeps.lut16_cases())
N_LUT16S = sum(1 for _ in sweeps.lut16s_cases())
N_SIGNMAG8 = sum(1 for _ in sweeps.signmag8_cases())


@pytest.mark.parametrize("case", range(N_LUT16))
def test_lut16_sweep_numpy_and_c_equal_integer_argmin(case):
    name, w, s, L = list(sweeps.lut16_cases())[case]
    want = exact.lut16_exact_indices(w, s, L)
    got = lut16.indices(w, s, L)
    assert np.array_equal(got, want), name
    assert np.array_equal(native.lut16_indices(w, s, L), want), name


@pytest.mark.parametrize("case", range(N_LUT16S))
def test_lut16s_sweep_numpy_and_c_equal_integer_argmin(case):
    name, w, s, T = list(sweeps.lut16s_cases())[case]
    tables = np.ascontiguousarray(np.broadcast_to(T, (w.shape[0], 1, 16)))
    want = exact.lut16_exact_indices(w, s, tables)
    assert np.array_equal(lut16.indices(w, s, tables), want), name
    assert np.array_equal(native.lut16_indices(w, s, tables), want), name


@pytest.mark.parametrize("case", range(N_SIGNMAG8))
def test_signmag8_sweep_numpy_and_c_equal_integer_argmin(case):
    name, w, cb = list(sweeps.signmag8_cases())[case]
    want = exact.signmag8_exact_indices(w, cb)
    assert np.array_equal(signmag8.indices(w, cb), want), name
    assert np.array_equal(native.signmag8_indices(w, cb), want), name


def test_dyadic_sweep_c_equals_numpy():
    """The C dyadic quantizer (the GPU tests' checker) against the numpy
    oracle, which test_oracle_dyadic pins to exact-rational argmin, on the
    same every-value sweeps the GPU test runs."""
    for sb, w in sweeps.dyadic_cases():
        idx_c, s_c = native.dyadic_quantize(w)
        s_n = dyadic.scales(w)
        assert np.array_equal(s_c, s_n), hex(sb)
        assert np.array_equal(idx_c, dyadic.indices(w, s_n)), hex(sb)


def test_cases_where_rounded_distances_tie():
    """Constructed cases where a distance rounded to fp32 (and to fp64 for
    the widest gaps) cannot tell the nearest level: a tiny weight between a
    symmetric pair, a weight beyond the top level with levels in both
    orders, tiny levels ahead of unit ones."""
    def one(wv, levels_vals, scale=1.0):
        s = bits.rne_bf16(np.array([[scale]]))
        L = np.zeros((1, 1, 16), np.uint16)
        lv = bits.rne_bf16(np.asarray(levels_vals, np.float64))
        L[0, 0, :len(lv)] = lv
        L[0, 0, len(lv):] = lv[-1]
        w = np.zeros((1, 64), np.uint16)
        w[0, 0] = bits.rne_bf16(np.array([wv]))[0]
        want = exact.lut16_exact_indices(w, s, L)[0, 0]
        assert lut16.indices(w, s, L)[0, 0] == want
        assert native.lut16_indices(w, s, L)[0, 0] == want
        return want
    # tiny positive weight between -1 and +1 (in either order): +1 is nearer
    assert one(2.0 ** -120, [-1.0, 1.0]) == 1
    assert one(2.0 ** -120, [1.0, -1.0]) == 0
    assert one(-(2.0 ** -120), [1.0, -1.0]) == 1
    # a weight far above every level: the largest level is nearest
    assert one(2.0 ** 100, [0.5, 1.0, 0.25]) == 1
    assert one(2.0 ** 100, [1.0, 0.5], scale=2.0 ** -100) == 0
    # levels 2^-100 and 1 at distance ~0.5 from w = 0.5: the tiny level wins
    assert one(0.5, [1.0, 2.0 ** -100]) == 1
    assert one(0.5, [2.0 ** -100, 1.0]) == 0
    # an exact midpoint still goes to the lower index
    assert one(0.5, [1.0, 0.0]) == 0
    assert one(0.5, [0.0, 1.0]) == 0


def test_signmag8_infinite_magnitudes():
    """+inf magnitudes (the fit's output beyond the fp16 range) are never
    nearer than a finite one; a group of only +inf takes index 0."""
    w = np.zeros((1, 64), np.uint16)
    w[0, :4] = bits.rne_bf16(np.array([1e30, -1e30, 0.0, 65504.0]))
    cb = np.full((1, 2, 8), 0x7C00, np.uint16)
    cb[0, 0, 5] = bits.rne_fp16(np.array([2.0]))[0]
    want = exact.signmag8_exact_indices(w, cb)
    assert list(want[0, :4]) == [5, 13, 5, 5]
    assert np.all(want[0, 32:] == 0)
    assert np.array_equal(signmag8.indices(w, cb), want)
    assert np.array_equal(native.signmag8_indices(w, cb), want)
