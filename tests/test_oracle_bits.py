"""Pins for oracle/bits.py: bf16 / fp16 decode and round-to-nearest-even."""

from fractions import Fraction

import numpy as np
import torch

from oracle import bits
from tests import exact


def _random_values(n, seed):
    g = np.random.default_rng(seed)
    # wide exponent spread, including subnormal bf16 / fp16 ranges
    mant = g.random(n) + 0.5
    e = g.integers(-140, 128, n)
    v = np.ldexp(mant, e) * np.where(g.random(n) < 0.5, -1, 1)
    return v


def test_decode_matches_torch():
    b = bits.all_finite_bf16()
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bits.bf16_to_f64(b), t)
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 10) & 0x1F) != 0x1F]
    assert np.array_equal(bits.f16_to_f64(h), h.view(np.float16).astype(np.float64))


def test_decode_matches_hand_decoder():
    b = bits.all_finite_bf16()[::97]
    for x in b:
        assert Fraction(float(bits.bf16_to_f64(np.array([x]))[0])) == exact.bf16_fraction(x)


def test_rne_bf16_vs_exact_rational_random():
    v = _random_values(4000, 1)
    v = v[np.abs(v) < 3e38]
    got = bits.rne_bf16(v)
    for x, g in zip(v, got):
        want = exact.fraction_to_bf16_bits(exact.rne_bf16_fraction(Fraction(float(x))))
        if want == 0 and x < 0:
            want = 0x8000
        assert int(g) == want, (x, hex(int(g)), hex(want))


def test_rne_bf16_ties_to_even_and_subnormals():
    # exact halfway points between adjacent bf16 values: must go to the even one
    b = bits.all_finite_bf16()
    b = b[(b & 0x8000) == 0]
    b = b[b < 0x7F7F]
    lo = bits.bf16_to_f64(b)
    hi = bits.bf16_to_f64(b + 1)
    mid = (lo + hi) / 2          # exact in fp64
    got = bits.rne_bf16(mid)
    want = np.where(b % 2 == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # just above / below the midpoint
    assert np.array_equal(bits.rne_bf16(np.nextafter(mid, np.inf)), (b + 1).astype(np.uint16))
    assert np.array_equal(bits.rne_bf16(np.nextafter(mid, -np.inf)), b)


def test_rne_bf16_vs_bit_trick_on_fp32():
    # an independent method on fp32 inputs: add 0x7FFF + lsb and truncate
    g = np.random.default_rng(2)
    u = g.integers(0, 0x7F7F0000, 200000, dtype=np.uint32)
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    f = u.view(np.float32)
    trick = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(bits.rne_bf16(f.astype(np.float64)), trick)


def test_rne_bf16_overflow():
    mx = float(exact.bf16_fraction(0x7F7F))
    half_ulp = 2.0 ** (127 - 8)
    assert bits.rne_bf16(np.array([mx + half_ulp * 0.999]))[0] == 0x7F7F
    assert bits.rne_bf16(np.array([mx + half_ulp]))[0] == 0x7F80   # tie -> even -> inf


def test_rne_fp16_vs_numpy_and_exact():
    v = _random_values(20000, 3)
    v = v[np.abs(v) < 65000]
    # numpy converts float64 -> float16 with one correct rounding
    assert np.array_equal(bits.rne_fp16(v), v.astype(np.float16).view(np.uint16))
    for x in v[:500]:
        want = exact.rne_fp16_fraction(Fraction(float(x)))
        assert Fraction(float(bits.f16_to_f64(bits.rne_fp16(np.array([x])))[0])) == want
