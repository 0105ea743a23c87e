"""Pins for oracle/matmul.py: the fp64 GEMV/GEMM reference and its bound."""

from fractions import Fraction

import numpy as np

import synthetic
from oracle import bits, dyadic, matmul, native
from tests import exact


def test_gemm_ref_vs_exact_dot_products():
    x = synthetic.normal_bf16((3, 128), 1.0, 41)
    w = synthetic.normal_bf16((5, 128), 0.02, 42)
    wv = bits.bf16_to_f64(w)
    y, b = matmul.gemm_ref(x, wv)
    assert y.shape == (3, 5)
    for i in range(3):
        for n in range(5):
            prods = [exact.bf16_fraction(x[i, k]) * exact.bf16_fraction(w[n, k]) for k in range(128)]
            ye = sum(prods, Fraction(0))
            be = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(y[i, n]) - ye) <= be * Fraction(1, 2 ** 45)
            assert abs(Fraction(b[i, n]) - be) <= be * Fraction(1, 2 ** 45)


def test_unit_vector_selects_a_column():
    w = synthetic.normal_bf16((16, 256), 0.02, 43)
    p, s = dyadic.quantize_pack(w)
    wh = bits.bf16_to_f64(dyadic.dequant(p, s))
    x = np.zeros((1, 256), np.uint16)
    x[0, 77] = 0x3F80
    y, _ = matmul.gemm_ref(x, wh)
    assert np.array_equal(y[0], wh[:, 77])


def test_tolerance_rule():
    y_ref = np.array([1.0, -2.0, 0.0])
    bound = np.array([10.0, 10.0, 10.0])
    assert matmul.within_tolerance(y_ref + 0.0099, y_ref, bound).all()
    assert not matmul.within_tolerance(y_ref + 0.0102, y_ref, bound).any()
    assert matmul.within_tolerance(np.array([0, 0, 9e-7]), np.zeros(3), np.zeros(3)).all()
    # bf16 output adds one output rounding
    assert matmul.within_tolerance([1.0 + 2 ** -8], [1.0], [0.0], bf16_out=True).all()


def test_c_dyadic_matmul_equals_numpy_reference():
    """The C oracle's fused dequant + fp64 matmul (timed by the benchmark's CPU
    baseline) against dequant + gemm_ref: both are fp64 sums of the same exact
    products, so they differ only by fp64 summation order, far below 2**-40 of
    the absolute sum; a zero-weight row and a unit vector are exact."""
    for n, k, m, seed in ((37, 320, 1, 1), (64, 1024, 5, 2), (5, 64, 16, 3)):
        w = synthetic.student_t_bf16((n, k), 4, 0.02, 50 + seed)
        w[0, :] = 0
        x = synthetic.normal_bf16((m, k), 1.0, 60 + seed)
        x[0, :] = 0
        x[0, k // 3] = 0x3F80
        p, s = dyadic.quantize_pack(w)
        wh = bits.bf16_to_f64(dyadic.dequant(p, s))
        want, bound = matmul.gemm_ref(x, wh)
        got = native.dyadic_matmul(p, s, x)
        assert np.all(np.abs(got - want) <= bound * 2.0 ** -40)
        assert np.array_equal(got[0], wh[:, k // 3]) and np.all(got[:, 0] == 0)
