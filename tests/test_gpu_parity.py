"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bit-exact for scales, packed bytes and dequantized values; GEMV / GEMM within
|y - y_ref| <= 1e-3 * sum|x w_hat| + 1e-6 of the fp64 oracle on the same
dequantized weights (plus one bf16 output rounding for bf16 outputs).  Sizes
span several tiles and a ragged tail; the full-size workloads are covered in
test_gpu_fullsize.py.
"""

import numpy as np
import pytest
import torch

import synthetic
from oracle import bits, dyadic, dyadic5, lut16, matmul, native, packing, signmag8, warmstart
from tests import sweeps
from tests.gpu_util import dev_bf16, dev_f16, dev_u8, host_bits, host_f32, host_u8, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import weight_only_bit_unpack_amd as m
    return m


def _edge_weight(n, k, seed, huge=True):
    """Gaussian weight with planted edge cases: an all-zero group, -0.0,
    subnormal-scale and huge-scale groups, exact code midpoints, +-absmax.
    huge=False keeps every scale below 2**110 so that fp32 sums of products
    with N(0, 1) activations cannot overflow."""
    w = synthetic.normal_bf16((n, k), 0.02, seed)
    g = np.random.default_rng(seed)
    if n >= 6 and k >= 128:
        w[0, :64] = 0
        w[0, 64:128] = 0x8000
        w[1, :64] = (g.integers(0, 0x7F, 64) | (g.integers(0, 2, 64) << 15)).astype(np.uint16)
        w[2, :64] = (g.integers(0x7E00, 0x7F7F, 64)).astype(np.uint16)     # scale ~ 2^125
        if not huge:
            w[2, :64] = (g.integers(0x7600, 0x7700, 64)).astype(np.uint16)
        w[2, 64:128] = (g.integers(0x7600, 0x7700, 64)).astype(np.uint16)  # scale ~ 2^109
        w[3, :64] = np.tile(np.array([0x3F80, 0xBF80, 0x3F00, 0x3E80], np.uint16), 16)
        # midpoints (2t-15)/16 of scale 1.0, all exactly representable
        mids = bits.rne_bf16((2 * np.arange(15) - 15) / 16.0)
        w[4, :15] = mids
        w[4, 15] = 0x3F80
        w[5, 64:128] = (g.integers(0x0080, 0x0400, 64)).astype(np.uint16)  # tiny normal scale
    return w


# ------------------------------------------------------------------ DYADIC
@pytest.mark.parametrize("n,k", [(2048, 2048), (37, 320), (6, 128), (1, 64)])
def test_dyadic_quantize_pack_bitexact(w4, n, k):
    report("dyadic_quantize", n=n, k=k)
    w = _edge_weight(n, k, 100 + n)
    p, s = w4.w4_quantize_pack(dev_bf16(w), w4.W4_DYADIC)
    torch.cuda.synchronize()
    idx_o, s_o = native.dyadic_quantize(w)
    assert np.array_equal(host_bits(s), s_o)
    assert np.array_equal(host_u8(p), packing.pack(idx_o))
    if n * k <= 1 << 16:   # the numpy oracle itself on the small ones
        p2, s2 = dyadic.quantize_pack(w)
        assert np.array_equal(host_u8(p), p2) and np.array_equal(host_bits(s), s2)


def test_dyadic_quantize_exhaustive_values(w4):
    """Every finite bf16 value of magnitude <= s, both signs, in groups whose
    absmax is s, for scales with plain, full and sparse mantissas, the
    smallest subnormal and normal, the largest finite value and huge and tiny
    exponents: indices and scales bit-exact against the C oracle, which the
    CPU tests check against the numpy oracle on these same inputs
    (tests/sweeps.py; the numpy oracle is pinned to exact-rational argmin)."""
    report("dyadic_quantize_exhaustive")
    for sb, w in sweeps.dyadic_cases():
        p, s = w4.w4_quantize_pack(dev_bf16(w), w4.W4_DYADIC)
        torch.cuda.synchronize()
        idx_o, s_o = native.dyadic_quantize(w)
        assert np.array_equal(host_bits(s), s_o), hex(sb)
        assert np.array_equal(host_u8(p), packing.pack(idx_o)), hex(sb)


def test_dyadic5_quantize_exhaustive_values(w4):
    """DYADIC5 at widths 3, 4 and 5: every finite bf16 value of magnitude <= s
    in groups of absmax s, for the same kinds of scales as the 4-bit test."""
    report("dyadic5_quantize_exhaustive")
    for sb in (0x3F80, 0x3FFF, 0x3C23, 0x0001, 0x0080, 0x7F7F, 0x7A01):
        w = sweeps.groups_with_absmax(sb, 64)
        widths = np.resize(np.array([3, 4, 5], np.uint8), (w.shape[0], 1))
        p, m, s = w4.w4_quantize_dyadic5(dev_bf16(w), dev_u8(widths))
        torch.cuda.synchronize()
        idx5, s_o = dyadic5.quantize(w, widths)
        nib, hi = dyadic5.planes(idx5)
        assert np.array_equal(host_bits(s), s_o), hex(sb)
        assert np.array_equal(host_u8(p), nib), hex(sb)
        assert np.array_equal(host_u8(m), hi), hex(sb)


def test_lut16_quantize_exhaustive_values(w4):
    """LUT16 and LUT16S exact nearest level: every finite bf16 weight against
    sorted tables (with and without duplicated levels), the uniform grid
    whose every midpoint is a bf16 weight (exact ties), tables with levels
    far apart in magnitude, symmetric pairs and unsorted entries beyond
    [-1, 1], under scales from the smallest subnormal to the largest finite
    bf16 (tests/sweeps.py; the CPU tests pin the C checker to integer brute
    force on exactly these inputs).  Sorted distinct tables take the kernel's
    midpoint count, the others its distance scan."""
    report("lut16_quantize_exhaustive")
    for name, w, s, L in sweeps.lut16_cases():
        p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_LUT16, scales=dev_bf16(s),
                                   codebook=dev_bf16(L))
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(p), packing.pack(native.lut16_indices(w, s, L))), name
    for name, w, s, T in sweeps.lut16s_cases():
        p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_LUT16S, scales=dev_bf16(s),
                                   codebook=dev_bf16(T))
        torch.cuda.synchronize()
        tables = np.ascontiguousarray(np.broadcast_to(T, (w.shape[0], 1, 16)))
        assert np.array_equal(host_u8(p), packing.pack(native.lut16_indices(w, s, tables))), name


def test_lut16_dequant_extreme_scales_and_tables(w4):
    """RNE_bf16(s * L) for every index, tables with entries beyond [-1, 1]
    (the call takes any finite bf16 table), signed zeros and subnormals,
    under scales from the smallest subnormal to the largest finite bf16
    (products that overflow to +-inf, round to the largest finite value or
    underflow): LUT16 and LUT16S against the oracle, bit for bit."""
    report("lut16_dequant_extreme")
    g = np.random.default_rng(73)
    scales = np.array([0x0001, 0x0080, 0x3F80, 0x7F7F, 0x7F00, 0x4000, 0x00FF, 0x3C23], np.uint16)
    G = 64 * len(scales)
    idx = np.tile(np.arange(16, dtype=np.uint8), 4)[None, :].repeat(G, axis=0)   # [G, 64]
    L = g.choice(np.array([0x3F80, 0xBF80, 0x4000, 0xC0F0, 0x0000, 0x8000, 0x0001, 0x8040,
                           0x3F7F, 0x3FFF, 0x7F7F, 0x0080], np.uint16), size=(G, 1, 16))
    L[:, 0, 5] = bits.rne_bf16(g.uniform(-4, 4, G))
    s = np.repeat(scales, 64)[:, None].astype(np.uint16)
    pk = dev_u8(packing.pack(idx))
    out = w4.w4_unpack_dequant(pk, w4.W4_LUT16, scales=dev_bf16(s), codebook=dev_bf16(L))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), lut16.dequant_from_indices(idx, s, L))
    T = np.ascontiguousarray(L[7, 0])
    out = w4.w4_unpack_dequant(pk, w4.W4_LUT16S, scales=dev_bf16(s), codebook=dev_bf16(T))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), lut16.dequant_from_indices(
        idx, s, np.ascontiguousarray(np.broadcast_to(T, L.shape))))


def test_signmag8_quantize_exhaustive_values(w4):
    """SIGNMAG8 sign + exact nearest magnitude: every finite bf16 weight
    against codebooks with subnormal, duplicated, zero, unsorted, maximal
    (65504) and +inf fp16 magnitudes, and the grid j / 8 whose midpoints are
    bf16 weights (tests/sweeps.py, pinned on the CPU)."""
    report("signmag8_quantize_exhaustive")
    for name, w, cb in sweeps.signmag8_cases():
        p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(p), packing.pack(native.signmag8_indices(w, cb))), name


@pytest.mark.parametrize("n,k", [(2048, 2048), (37, 320), (6, 128)])
def test_dyadic_dequant_bitexact(w4, n, k):
    report("dyadic_dequant", n=n, k=k)
    w = _edge_weight(n, k, 200 + n)
    p_o, s_o = dyadic.quantize_pack(w) if n * k <= 1 << 16 else (None, None)
    if p_o is None:
        idx, s_o = native.dyadic_quantize(w)
        p_o = packing.pack(idx)
    out = w4.w4_unpack_dequant(dev_u8(p_o), w4.W4_DYADIC, scales=dev_bf16(s_o))
    torch.cuda.synchronize()
    want = native.dyadic_dequant(packing.unpack(p_o), s_o)
    assert np.array_equal(host_bits(out), want)


def test_dyadic_dequant_exhaustive_scales(w4):
    """Every finite bf16 scale of either sign x every index, on the GPU (a
    caller may pass its own scales; code 8 rebuilds to +0 for every scale,
    also for the negative ones of 2**120 and more, which take the wide
    rebuild).  Rows are ordered so that waves mix plain and wide scales."""
    allb = bits.all_finite_bf16()
    n = len(allb)
    idx = np.tile(np.arange(16, dtype=np.uint8), (n, 4))
    report("dyadic_dequant_exhaustive", n=n)
    out = w4.w4_unpack_dequant(dev_u8(packing.pack(idx)), w4.W4_DYADIC, scales=dev_bf16(allb[:, None]))
    torch.cuda.synchronize()
    got = host_bits(out)
    assert np.array_equal(got, dyadic.dequant_from_indices(idx, allb[:, None]))
    assert np.all(got[:, 8::16] == 0)


def _gemv_check(y, x_bits, w_hat, bf16_out):
    y_ref, bound = matmul.gemm_ref(x_bits, w_hat)
    ok = matmul.within_tolerance(host_f32(y), y_ref, bound, bf16_out=bf16_out)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError(f"{(~ok).sum()} outside tolerance, e.g. {bad.tolist()} "
                             f"got {host_f32(y)[tuple(bad[0])]} want {y_ref[tuple(bad[0])]}")


# m > 1 on few row tiles: while the m x k activations fit one block's LDS,
# 16-row tiles with k split between a block's waves ((37, 320, 3) ragged,
# (300, 1024, 4 and 16), (130, 2944, 7), (40000, 128, 2)); else k split across
# blocks (k slices, partial sums added in order by a second kernel): (37,
# 20800, 3) has a ragged last slice, (70, 49472, 16) more activations per
# slice than fit in LDS (chunks inside a slice), (64, 4096, 16) even slices,
# (33, 65600, 2) many.  (33, 65600, 1) takes k in three chunks inside each
# block (the last one ragged).
@pytest.mark.parametrize("n,k,m", [(2048, 2048, 1), (37, 320, 1), (37, 320, 3), (300, 1024, 4),
                                   (300, 1024, 16), (64, 4096, 16), (40000, 128, 2),
                                   (70000, 64, 1), (70, 49472, 16), (130, 2944, 7),
                                   (33, 65600, 1), (33, 65600, 2), (37, 20800, 3)])
@pytest.mark.parametrize("ybf16", [False, True])
def test_dyadic_gemv(w4, n, k, m, ybf16):
    report("dyadic_gemv", n=n, k=k, m=m, ybf16=ybf16)
    w = _edge_weight(n, k, 300 + n + k, huge=False)
    idx, s = native.dyadic_quantize(w)
    p = packing.pack(idx)
    x = synthetic.normal_bf16((m, k), 1.0, 301 + m)
    y = w4.w4_gemv(dev_u8(p), dev_bf16(x), w4.W4_DYADIC, scales=dev_bf16(s),
                   y_dtype=torch.bfloat16 if ybf16 else torch.float32)
    torch.cuda.synchronize()
    w_hat = bits.bf16_to_f64(native.dyadic_dequant(idx, s))
    _gemv_check(y, x, w_hat, ybf16)


def test_dyadic_gemv_unit_vectors_exact(w4):
    n, k = 96, 512
    report("dyadic_gemv_unit", n=n, k=k)
    w = _edge_weight(n, k, 401, huge=False)
    idx, s = native.dyadic_quantize(w)
    p = dev_u8(packing.pack(idx))
    sd = dev_bf16(s)
    w_hat = bits.bf16_to_f64(native.dyadic_dequant(idx, s))
    w_hat[~np.isfinite(w_hat)] = 0
    for col in [0, 1, 63, 64, 255, 256, 511]:
        x = np.zeros((1, k), np.uint16)
        x[0, col] = 0x3F80
        y = host_f32(w4.w4_gemv(p, dev_bf16(x), w4.W4_DYADIC, scales=sd))
        assert np.array_equal(y[0], w_hat[:, col]), col
    # all-index-8 weights give exactly zero
    z = w4.w4_gemv(dev_u8(np.full((n, k // 2), 0x88, np.uint8)), dev_bf16(x), w4.W4_DYADIC, scales=sd)
    assert torch.count_nonzero(z).item() == 0


_EXTREME_SCALES = np.array([0x0001, 0x0080, 0x00FF, 0x3C23, 0x3F80, 0x4000, 0x7E55, 0x7F7F],
                           np.uint16)


def _extreme_codec_case(codec, n, k, seed):
    """Random indices with side data at the extremes of bf16 / fp16 (scales
    from the smallest subnormal to the largest finite bf16, table entries at
    +-1, +-0 and subnormal, magnitudes up to 65504): (packed, side tables,
    fp64 dequantized weight).  Every dequantized value is finite."""
    g = np.random.default_rng(seed)
    s = g.choice(_EXTREME_SCALES, size=(n, k // 64))
    if codec == 0:
        idx = g.integers(0, 16, (n, k)).astype(np.uint8)
        return (packing.pack(idx), dict(scales=dev_bf16(s)),
                bits.bf16_to_f64(dyadic.dequant_from_indices(idx, s)))
    if codec in (1, 3):
        kinds = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x0001, 0x8001, 0x3F7F, 0xBE00],
                         np.uint16)
        L = g.choice(kinds, size=(n, k // 64, 16))
        L[..., :4] = bits.rne_bf16(g.uniform(-1, 1, (n, k // 64, 4)))
        idx = g.integers(0, 16, (n, k)).astype(np.uint8)
        if codec == 3:
            T = np.ascontiguousarray(L[0, 0])
            tables = np.ascontiguousarray(np.broadcast_to(T, L.shape))
            return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(T)),
                    bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables)))
        return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(L)),
                bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, L)))
    if codec == 4:
        idx5 = g.integers(0, 32, (n, k)).astype(np.uint8)
        nib, msb = dyadic5.planes(idx5)
        return (nib, dict(scales=dev_bf16(s), codebook=dev_u8(msb)),
                bits.bf16_to_f64(dyadic5.dequant_from_indices(idx5, s)))
    cb = g.choice(np.array([0x7BFF, 0x0001, 0x0000, 0x3C00, 0x03FF, 0x0400, 0x5A5A], np.uint16),
                  size=(n, k // 32, 8))
    nib = g.integers(0, 16, (n, k)).astype(np.uint8)
    return packing.pack(nib), dict(codebook=dev_f16(cb)), signmag8.dequant_values(cb, nib)


@pytest.mark.parametrize("codec", [0, 1, 2, 3, 4])
def test_unit_vectors_extreme_side_data(w4, codec):
    """x = rows of the identity: every output is one rebuilt weight times 1.0
    plus products with 0, so the GEMV (m = 16) and the GEMM (m = 128) must
    return the dequantized weights exactly, for every codec's rebuild at the
    extremes of its side data (the matrix kernels rebuild on their own, apart
    from the dequant kernel)."""
    n, k = 64, 128
    report("unit_vectors_extreme", codec=codec)
    p, side, w_hat = _extreme_codec_case(codec, n, k, 1700 + codec)
    pk = dev_u8(p)
    for c0 in range(0, k, 16):
        x = np.zeros((16, k), np.uint16)
        x[np.arange(16), c0 + np.arange(16)] = 0x3F80
        y = host_f32(w4.w4_gemv(pk, dev_bf16(x), codec, **side))
        assert np.array_equal(y, w_hat[:, c0:c0 + 16].T), (codec, c0)
    x = np.zeros((128, k), np.uint16)
    x[np.arange(128), np.arange(128)] = 0x3F80
    y = host_f32(w4.w4_gemm(pk, dev_bf16(x), codec, **side))
    assert np.array_equal(y, w_hat.T), codec


@pytest.mark.parametrize("op", ["gemv", "gemm"])
def test_dyadic_wide_scales(w4, op):
    """Scales >= 2**120 take the wide rebuild; activations ~2**-20 keep the
    fp32 sums finite."""
    n, k = 64, 256
    report("dyadic_wide", op=op)
    w = _edge_weight(n, k, 402)
    w[10:20, :] = (np.random.default_rng(3).integers(0x7C00, 0x7F7F, (10, k))
                   | (np.random.default_rng(4).integers(0, 2, (10, k)) << 15)).astype(np.uint16)
    idx, s = native.dyadic_quantize(w)
    x = bits.rne_bf16(bits.bf16_to_f64(synthetic.normal_bf16((2, k), 1.0, 403)) * 2.0 ** -20)
    fn = w4.w4_gemv if op == "gemv" else w4.w4_gemm
    y = fn(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_DYADIC, scales=dev_bf16(s))
    torch.cuda.synchronize()
    _gemv_check(y, x, bits.bf16_to_f64(native.dyadic_dequant(idx, s)), False)


@pytest.mark.parametrize("m", [1, 16])
def test_dyadic_gemv_deterministic(w4, m):
    n, k = 4096, 2048
    w = synthetic.normal_bf16((n, k), 0.02, 402)
    x = dev_bf16(synthetic.normal_bf16((m, k), 1.0, 403))
    p, s = w4.w4_quantize_pack(dev_bf16(w), w4.W4_DYADIC)
    a = w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s)
    b = w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dyadic_gemv_batched(w4):
    shapes = [(2048, 2048), (5632, 2048), (2048, 5632), (100, 320), (64, 64)]
    report("dyadic_gemv_batched", count=len(shapes))
    probs, refs = [], []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16((n, k), 4, 0.02, 500 + i)
        x = synthetic.normal_bf16((1, k), 1.0, 600 + i)
        idx, s = native.dyadic_quantize(w)
        p = packing.pack(idx)
        y = torch.full((1, n), float("nan"), device="cuda")
        probs.append({"packed": dev_u8(p), "scales": dev_bf16(s), "x": dev_bf16(x), "y": y})
        refs.append((x, bits.bf16_to_f64(native.dyadic_dequant(idx, s))))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_DYADIC)
    batch()
    batch()
    torch.cuda.synchronize()
    for pr, (x, w_hat) in zip(probs, refs):
        _gemv_check(pr["y"], x, w_hat, False)


@pytest.mark.parametrize("n,k,m", [(200, 576, 1), (200, 576, 130), (1024, 2048, 256), (64, 64, 128),
                                   (100, 65600, 130), (64, 128, 1), (300, 1152, 100),
                                   (200, 640, 128), (130, 256, 257), (100, 65536, 120)])
def test_dyadic_gemm(w4, n, k, m):
    report("dyadic_gemm", n=n, k=k, m=m)
    w = _edge_weight(n, k, 700 + n, huge=False)
    idx, s = native.dyadic_quantize(w)
    x = synthetic.normal_bf16((m, k), 1.0, 701 + m)
    y = w4.w4_gemm(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_DYADIC, scales=dev_bf16(s))
    torch.cuda.synchronize()
    _gemv_check(y, x, bits.bf16_to_f64(native.dyadic_dequant(idx, s)), False)


# ------------------------------------------------------------------ LUT16
def _lut_case(n, k, seed):
    w = synthetic.normal_outliers_bf16((n, k), 0.015, 0.001, 0.15, seed)
    if n >= 2:
        w[1, :64] = 0
    s, L = native.lut16_fit(w)
    return w, s, L


@pytest.mark.parametrize("n,k", [(512, 1024), (37, 320)])
def test_lut16_quantize_dequant_bitexact(w4, n, k):
    report("lut16_quant_dequant", n=n, k=k)
    w, s, L = _lut_case(n, k, 800 + n)
    p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_LUT16, scales=dev_bf16(s), codebook=dev_bf16(L))
    torch.cuda.synchronize()
    idx = native.lut16_indices(w, s, L)
    assert np.array_equal(host_u8(p), packing.pack(idx))
    if n * k <= 1 << 16:
        assert np.array_equal(host_u8(p), lut16.quantize_pack(w, s, L))
    out = w4.w4_unpack_dequant(dev_u8(packing.pack(idx)), w4.W4_LUT16, scales=dev_bf16(s),
                               codebook=dev_bf16(L))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), lut16.dequant_from_indices(idx, s, L))


@pytest.mark.parametrize("iters", [0, 1, 25])
def test_lut16_fit_bitexact(w4, iters):
    """GPU k-means LUT fit == the C oracle's fit, bit for bit: tie-heavy groups
    (signed-zero runs, few distinct values, all-zero, subnormal and near-max
    magnitudes) and Gaussian-with-outliers groups, 16 groups per block with a
    ragged last block."""
    from tests.test_oracle_lut16 import tie_groups
    report("lut16_fit", iters=iters)
    ties = tie_groups().reshape(1, 8 * 64)
    rnd = synthetic.normal_outliers_bf16((37, 320), 0.015, 0.001, 0.15, 77)
    for w in (ties, rnd, synthetic.normal_bf16((300, 1024), 0.02, 78), rnd[:1, :64]):
        s_o, L_o = native.lut16_fit(w, iters)
        s, L = w4.w4_lut16_fit(dev_bf16(w), iters)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(s), s_o), w.shape
        assert np.array_equal(host_bits(L), L_o), w.shape


@pytest.mark.parametrize("iters", [0, 1, 25])
def test_signmag8_fit_bitexact(w4, iters):
    """GPU k-means magnitude fit == the C oracle's fit, bit for bit: tie and
    fp16-rounding groups (equal magnitudes, signed zeros, subnormal, overflow),
    Student-t groups, 32 groups per block with a ragged last block, k a
    multiple of 32 but not of 64."""
    from tests.test_oracle_lut16 import signmag8_tie_groups
    report("signmag8_fit", iters=iters)
    ties = signmag8_tie_groups()
    rnd = synthetic.student_t_bf16((37, 352), 5, 0.02, 79)
    for w in (ties, rnd, synthetic.normal_bf16((300, 1024), 0.02, 80), rnd[:1, :32]):
        cb_o = native.signmag8_fit(w, iters)
        cb = w4.w4_signmag8_fit(dev_bf16(w), iters)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(cb), cb_o), w.shape


def _warm_check(w, cb, params, iters, max_mismatch):
    """GPU warm-start fit against the oracle.  Chosen candidates: equal, or a
    near-tie of the oracle's own candidate errors (relative 1e-9, or 1e-28
    gmax^2 absolute), on at most
    max_mismatch of the groups; codebooks: bit-identical wherever the chosen
    candidates are; elsewhere the GPU's levels, used as a codebook, do no
    worse than its chosen candidate's start (up to fp16 rounding)."""
    a = np.abs(bits.bf16_to_f64(w)).reshape(-1, 32)
    lev, code_o, sses = warmstart.warm_start(a)
    M_o = bits.rne_fp16(lut16.lloyd(a, lev, iters))
    code_g = np.asarray(params).reshape(-1) if isinstance(params, np.ndarray) else \
        host_u8(params).reshape(-1)
    M_g = np.asarray(cb).reshape(-1, 8) if isinstance(cb, np.ndarray) else \
        host_bits(cb).reshape(-1, 8)
    index = {c[0]: i for i, c in enumerate(warmstart.candidates())}
    live = a.max(axis=-1) > 0
    assert np.all(code_g[~live] == 0) and np.all(M_g[~live] == 0)
    gi = np.array([index[int(c)] for c in code_g])
    s_g = sses[np.arange(a.shape[0]), gi]
    s_min = sses.min(axis=-1)
    # a near-tie: relative 1e-9, or a few ulps of gmax in every level (an exact
    # zero error on one side can be 1e-32 * gmax^2 on the other)
    slack = s_min * 1e-9 + 1e-28 * a.max(axis=-1) ** 2
    assert np.all(s_g[live] <= (s_min + slack)[live]), "GPU picked a worse candidate"
    same = code_g == code_o
    assert np.array_equal(M_g[same], M_o[same])
    diff = ~same
    print(f"  {a.shape[0]} groups, {int(diff.sum())} with another near-tie candidate")
    assert diff.sum() <= max_mismatch * a.shape[0], diff.sum()
    if diff.any():
        e_g = warmstart.group_sse(a[diff], bits.f16_to_f64(M_g[diff]))
        assert np.all(e_g <= s_g[diff] * (1 + 2.0 ** -9) + 1e-30)


@pytest.mark.parametrize("iters", [0, 25])
def test_signmag8_fit_warm(w4, iters):
    """Warm-start magnitude fit (112 transforms, then Lloyd) on the GPU vs the
    oracle: tie and fp16-rounding groups (equal magnitudes, signed zeros,
    subnormals, overflow; near-ties of candidates allowed there), Student-t
    and Gaussian groups with a ragged last block and k a multiple of 32 only."""
    from tests.test_oracle_lut16 import signmag8_tie_groups
    report("signmag8_fit_warm", iters=iters)
    ties = signmag8_tie_groups()
    cb, pr = w4.w4_signmag8_fit_warm(dev_bf16(ties), iters)
    torch.cuda.synchronize()
    _warm_check(ties, cb, pr, iters, max_mismatch=1.0)
    for w in (synthetic.student_t_bf16((37, 352), 5, 0.02, 81),
              synthetic.normal_bf16((8, 1024), 0.02, 82)):
        cb, pr = w4.w4_signmag8_fit_warm(dev_bf16(w), iters)
        torch.cuda.synchronize()
        _warm_check(w, cb, pr, iters, max_mismatch=0.01)


@pytest.mark.parametrize("m", [1, 4, 16, 200])
def test_lut16_gemv_and_gemm(w4, m):
    """GEMV for m <= 16; GEMM at every m (128-row blocks for m <= 128,
    256-row blocks for m = 200)."""
    n, k = 300, 1024
    report("lut16_gemv", n=n, k=k, m=m)
    w, s, L = _lut_case(n, k, 900 + m)
    idx = native.lut16_indices(w, s, L)
    w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, L))
    x = synthetic.normal_bf16((m, k), 1.0, 901 + m)
    args = dict(scales=dev_bf16(s), codebook=dev_bf16(L))
    if m <= 16:
        y = w4.w4_gemv(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_LUT16, **args)
        torch.cuda.synchronize()
        _gemv_check(y, x, w_hat, False)
    y2 = w4.w4_gemm(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_LUT16, **args)
    torch.cuda.synchronize()
    _gemv_check(y2, x, w_hat, False)


@pytest.mark.parametrize("m", [1, 16, 17, 256])
def test_linear_dispatch(w4, m):
    """w4_linear equals the call it selects, bit for bit, on both sides of m = 16."""
    n, k = 300, 1024
    report("linear", m=m)
    w = synthetic.normal_bf16((n, k), 0.02, 1700 + m)
    x = dev_bf16(synthetic.normal_bf16((m, k), 1.0, 1701 + m))
    p, s = w4.w4_quantize_pack(dev_bf16(w), w4.W4_DYADIC)
    y = w4.w4_linear(p, x, w4.W4_DYADIC, scales=s)
    direct = (w4.w4_gemv if m <= 16 else w4.w4_gemm)(p, x, w4.W4_DYADIC, scales=s)
    torch.cuda.synchronize()
    assert torch.equal(y, direct)


# ------------------------------------------------------------------ LUT16S
def _lut16s_case(n, k, seed):
    """Weight with a zero group, its group scales and the oracle's whole-weight
    table, the table repeated per group, and the oracle's indices."""
    w = synthetic.normal_outliers_bf16((n, k), 0.015, 0.001, 0.15, seed)
    w[0, :64] = 0
    s, T = lut16.fit_shared(w, iters=10)
    tables = np.ascontiguousarray(lut16.shared_tables(s, T))
    return w, s, T, tables, native.lut16_indices(w, s, tables)


@pytest.mark.parametrize("n,k", [(300, 1024), (37, 320)])
def test_lut16s_quantize_dequant_bitexact(w4, n, k):
    report("lut16s_quant", n=n, k=k)
    w, s, T, tables, idx = _lut16s_case(n, k, 950 + n)
    args = dict(scales=dev_bf16(s), codebook=dev_bf16(T))
    p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_LUT16S, **args)
    d = w4.w4_unpack_dequant(p, w4.W4_LUT16S, **args)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(p), packing.pack(idx))
    assert np.array_equal(host_bits(d), lut16.dequant_from_indices(idx, s, tables))


@pytest.mark.parametrize("m", [1, 4, 16, 100, 300])
def test_lut16s_matmul(w4, m):
    """GEMV (m <= 16: single call, fp32 and bf16 y) or GEMM (m = 100: 128-row
    blocks; m = 300: 256-row blocks)."""
    n, k = 300, 1024
    report("lut16s_matmul", n=n, k=k, m=m)
    w, s, T, tables, idx = _lut16s_case(n, k, 960 + m)
    w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables))
    x = synthetic.normal_bf16((m, k), 1.0, 961 + m)
    args = dict(scales=dev_bf16(s), codebook=dev_bf16(T))
    fn = w4.w4_gemv if m <= 16 else w4.w4_gemm
    y = fn(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_LUT16S, **args)
    yb = fn(dev_u8(packing.pack(idx)), dev_bf16(x), w4.W4_LUT16S, y_dtype=torch.bfloat16, **args)
    torch.cuda.synchronize()
    _gemv_check(y, x, w_hat, False)
    _gemv_check(yb, x, w_hat, True)


# ------------------------------------------------------------------ DYADIC5
def _d5_case(n, k, seed, huge=False):
    """Edge-case weight, random group widths (3, 4, 5 and two values that
    mean 5), the oracle's 5-bit indices, scales and both planes."""
    w = _edge_weight(n, k, seed, huge=huge)
    widths = np.random.default_rng(seed).choice([3, 4, 5, 0, 9], size=(n, k // 64)).astype(np.uint8)
    idx, s = dyadic5.quantize(w, widths)
    nib, msb = dyadic5.planes(idx)
    return w, widths, idx, s, nib, msb


@pytest.mark.parametrize("n,k", [(300, 1024), (37, 320), (6, 128)])
def test_dyadic5_quantize_dequant_bitexact(w4, n, k):
    """Per-group widths and widths = None (5 bits everywhere): scales, nibble
    plane and high-bit plane bit for bit; dequant of the oracle's planes."""
    report("dyadic5_quant", n=n, k=k)
    w, widths, idx, s, nib, msb = _d5_case(n, k, 1500 + n)
    for wd, want_idx in ((widths, idx), (None, dyadic5.indices(w, s))):
        p, m, sd = w4.w4_quantize_dyadic5(dev_bf16(w), None if wd is None else dev_u8(wd))
        torch.cuda.synchronize()
        want_nib, want_msb = dyadic5.planes(want_idx)
        assert np.array_equal(host_bits(sd), s)
        assert np.array_equal(host_u8(p), want_nib)
        assert np.array_equal(host_u8(m), want_msb)
    d = w4.w4_unpack_dequant(dev_u8(nib), w4.W4_DYADIC5, scales=dev_bf16(s), codebook=dev_u8(msb))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(d), dyadic5.dequant_from_indices(idx, s))


def test_dyadic5_dequant_exhaustive_scales(w4):
    """Every finite bf16 scale of either sign (zero included) x every 5-bit index."""
    allb = bits.all_finite_bf16()
    n = len(allb)
    idx = np.tile(np.arange(32, dtype=np.uint8), (n, 2))
    report("dyadic5_dequant_exhaustive", n=n)
    nib, msb = dyadic5.planes(idx)
    out = w4.w4_unpack_dequant(dev_u8(nib), w4.W4_DYADIC5, scales=dev_bf16(allb[:, None]),
                               codebook=dev_u8(msb))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), dyadic5.dequant_from_indices(idx, allb[:, None]))


@pytest.mark.parametrize("m", [1, 4, 16, 100, 300])
def test_dyadic5_matmul(w4, m):
    """GEMV (m <= 16: single call, k split for m > 1) or GEMM (m = 100: 128-row
    blocks; m = 300: 256-row blocks), fp32 and bf16 outputs, against the fp64
    oracle on the same 5-bit weights."""
    n, k = 300, 1024
    report("dyadic5_matmul", n=n, k=k, m=m)
    w, widths, idx, s, nib, msb = _d5_case(n, k, 1600 + m)
    w_hat = bits.bf16_to_f64(dyadic5.dequant_from_indices(idx, s))
    x = synthetic.normal_bf16((m, k), 1.0, 1601 + m)
    args = dict(scales=dev_bf16(s), codebook=dev_u8(msb))
    fn = w4.w4_gemv if m <= 16 else w4.w4_gemm
    y = fn(dev_u8(nib), dev_bf16(x), w4.W4_DYADIC5, **args)
    yb = fn(dev_u8(nib), dev_bf16(x), w4.W4_DYADIC5, y_dtype=torch.bfloat16, **args)
    torch.cuda.synchronize()
    _gemv_check(y, x, w_hat, False)
    _gemv_check(yb, x, w_hat, True)


# ------------------------------------------------------------------ SIGNMAG8
def _sm_case(n, k, seed):
    w = synthetic.student_t_bf16((n, k), 5, 0.02, seed)
    w[0, 0] = 0x8000
    cb = native.signmag8_fit(w)
    cb[0, 1, 0] = 0
    return w, cb


@pytest.mark.parametrize("n,k", [(512, 1024), (37, 320)])
def test_signmag8_quantize_dequant_bitexact(w4, n, k):
    report("signmag8_quant_dequant", n=n, k=k)
    w, cb = _sm_case(n, k, 1000 + n)
    p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    torch.cuda.synchronize()
    nib = native.signmag8_indices(w, cb)
    assert np.array_equal(host_u8(p), packing.pack(nib))
    if n * k <= 1 << 16:
        assert np.array_equal(host_u8(p), signmag8.quantize_pack(w, cb))
    out = w4.w4_unpack_dequant(dev_u8(packing.pack(nib)), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    assert np.array_equal(host_bits(out), signmag8.dequant_from_indices(nib, cb))


@pytest.mark.parametrize("m", [1, 5])
def test_signmag8_gemv_and_gemm(w4, m):
    n, k = 300, 1024
    report("signmag8_gemv", n=n, k=k, m=m)
    w, cb = _sm_case(n, k, 1100 + m)
    nib = native.signmag8_indices(w, cb)
    w_hat = signmag8.dequant_values(cb, nib)
    x = synthetic.normal_bf16((m, k), 1.0, 1101 + m)
    y = w4.w4_gemv(dev_u8(packing.pack(nib)), dev_bf16(x), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    torch.cuda.synchronize()
    _gemv_check(y, x, w_hat, False)
    y2 = w4.w4_gemm(dev_u8(packing.pack(nib)), dev_bf16(x), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    torch.cuda.synchronize()
    _gemv_check(y2, x, w_hat, False)


def _batched_case(codec, n, k, seed):
    """(packed, side tables, fp64 dequantized weight) of one batched problem."""
    if codec == 0:
        w = synthetic.student_t_bf16((n, k), 4, 0.02, seed)
        idx, s = native.dyadic_quantize(w)
        return packing.pack(idx), dict(scales=dev_bf16(s)), bits.bf16_to_f64(native.dyadic_dequant(idx, s))
    if codec == 1:
        w, s, L = _lut_case(n, k, seed)
        idx = native.lut16_indices(w, s, L)
        w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, L))
        return packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(L)), w_hat
    if codec == 4:
        w, widths, idx, s, nib, msb = _d5_case(n, k, seed)
        w_hat = bits.bf16_to_f64(dyadic5.dequant_from_indices(idx, s))
        return nib, dict(scales=dev_bf16(s), codebook=dev_u8(msb)), w_hat
    if codec == 3:
        w, s, T, tables, idx = _lut16s_case(n, k, seed)
        w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables))
        return packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(T)), w_hat
    w, cb = _sm_case(n, k, seed)
    nib = native.signmag8_indices(w, cb)
    return packing.pack(nib), dict(codebook=dev_f16(cb)), signmag8.dequant_values(cb, nib)


# every codec through the batched launch, ragged n, m > 1, repeated launches
@pytest.mark.parametrize("codec,m,shapes", [
    (0, 1, [(2048, 2048), (5632, 2048), (2048, 5632), (100, 1024), (70, 832)]),
    (0, 4, [(1000, 2048), (64, 1024), (333, 832)]),
    # m >= 5: the deeper activation staging (16 units in flight per thread),
    # with whole and partial last 256-k steps
    (0, 5, [(1000, 2048), (333, 832)]),
    (0, 6, [(130, 2880), (64, 256)]),
    (2, 12, [(300, 1024), (65, 2048), (77, 832)]),
    (1, 1, [(300, 1024), (129, 2048)]),
    (2, 3, [(300, 1024), (65, 2048)]),
    (3, 1, [(300, 1024), (129, 2048), (64, 64)]),
    (3, 16, [(300, 1024), (70, 832)]),
    (4, 1, [(2048, 2048), (300, 1024), (70, 832)]),
    (4, 8, [(300, 1024), (129, 2048)]),
    # m x k activations beyond one block's LDS: staged in k chunks
    (0, 16, [(300, 5632), (70, 2048), (130, 2880)]),
    (1, 16, [(200, 5632)]),
])
def test_gemv_batched_codecs(w4, codec, m, shapes):
    report("gemv_batched_codecs", codec=codec, m=m, count=len(shapes))
    probs, refs = [], []
    for i, (n, k) in enumerate(shapes):
        p, side, w_hat = _batched_case(codec, n, k, 1200 + 10 * codec + i)
        x = synthetic.normal_bf16((m, k), 1.0, 1300 + 10 * codec + i)
        y = torch.full((m, n), float("nan"), device="cuda")
        probs.append(dict(packed=dev_u8(p), x=dev_bf16(x), y=y, **side))
        refs.append((x, w_hat))
    batch = w4.w4_gemv_batched_plan(probs, codec)
    for rep in range(3):
        for pr in probs:
            pr["y"].fill_(float("nan"))
        batch()
        torch.cuda.synchronize()
        for pr, (x, w_hat) in zip(probs, refs):
            _gemv_check(pr["y"], x, w_hat, False)


# bf16 outputs of the batched launch: the m = 1 kernels at each tile height
# (64 rows for the first case, 16 for the small ones) and the m > 1 kernel
@pytest.mark.parametrize("codec,m,shapes", [
    (0, 1, [(2048, 2048), (5632, 2048), (70000, 256)]),
    (0, 1, [(300, 1024), (70, 832)]),
    (0, 5, [(300, 1024), (70, 832)]),
    (2, 1, [(300, 1024), (65, 2048)]),
    (3, 1, [(300, 1024), (129, 2048)]),
    (4, 2, [(300, 1024), (129, 2048)]),
])
def test_gemv_batched_bf16_output(w4, codec, m, shapes):
    report("gemv_batched_bf16", codec=codec, m=m, count=len(shapes))
    probs, refs = [], []
    for i, (n, k) in enumerate(shapes):
        p, side, w_hat = _batched_case(codec, n, k, 4200 + 10 * codec + i)
        x = synthetic.normal_bf16((m, k), 1.0, 4300 + 10 * codec + i)
        y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        probs.append(dict(packed=dev_u8(p), x=dev_bf16(x), y=y, **side))
        refs.append((x, w_hat))
    batch = w4.w4_gemv_batched_plan(probs, codec, y_dtype=torch.bfloat16)
    batch()
    torch.cuda.synchronize()
    for pr, (x, w_hat) in zip(probs, refs):
        _gemv_check(pr["y"], x, w_hat, True)


@pytest.mark.parametrize("m", [1, 4])
def test_gemv_batched_many_problems(w4, m):
    """More problems than a block's 256 threads look up in one round (the
    block -> problem search loops), including empty ones (n = 0), whose
    tiles are none."""
    g = np.random.default_rng(1400 + m)
    shapes = [(int(g.integers(1, 200)), int(g.choice([64, 128, 320]))) for _ in range(300)]
    shapes[7] = (0, 64)
    shapes[290] = (0, 128)
    report("gemv_batched_many", m=m, count=len(shapes))
    probs, refs = [], []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.normal_bf16((max(n, 1), k), 0.02, 1500 + i)[:n]
        x = synthetic.normal_bf16((m, k), 1.0, 1800 + i)
        idx, s = native.dyadic_quantize(np.ascontiguousarray(w))
        y = torch.full((m, n), float("nan"), device="cuda")
        probs.append({"packed": dev_u8(packing.pack(idx)) if n else torch.empty((0, k // 2), dtype=torch.uint8, device="cuda"),
                      "scales": dev_bf16(s) if n else torch.empty((0, k // 64), dtype=torch.bfloat16, device="cuda"),
                      "x": dev_bf16(x), "y": y})
        refs.append((x, bits.bf16_to_f64(native.dyadic_dequant(idx, s)) if n else None))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_DYADIC)
    batch()
    torch.cuda.synchronize()
    for pr, (x, w_hat) in zip(probs, refs):
        if w_hat is not None:
            _gemv_check(pr["y"], x, w_hat, False)


def _random_codec_case(codec, n, k, seed):
    """Random indices with ordinary side data (scales of Gaussian weights'
    groups, sorted tables in [-1, 1], fp16 magnitudes below 0.1): (packed,
    side tables, fp64 dequantized weight), cheap to build for many rows."""
    g = np.random.default_rng(seed)
    s = bits.rne_bf16(np.abs(g.normal(0.05, 0.01, (n, k // 64))))
    if codec == 0:
        idx = g.integers(0, 16, (n, k)).astype(np.uint8)
        return (packing.pack(idx), dict(scales=dev_bf16(s)),
                bits.bf16_to_f64(dyadic.dequant_from_indices(idx, s)))
    if codec in (1, 3):
        idx = g.integers(0, 16, (n, k)).astype(np.uint8)
        if codec == 3:
            T = bits.rne_bf16(np.sort(g.uniform(-1, 1, 16)))
            tables = np.ascontiguousarray(np.broadcast_to(T, (n, k // 64, 16)))
            return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(T)),
                    bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables)))
        L = bits.rne_bf16(np.sort(g.uniform(-1, 1, (n, k // 64, 16)), axis=-1))
        return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(L)),
                bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, L)))
    if codec == 4:
        idx5 = g.integers(0, 32, (n, k)).astype(np.uint8)
        nib, msb = dyadic5.planes(idx5)
        return (nib, dict(scales=dev_bf16(s), codebook=dev_u8(msb)),
                bits.bf16_to_f64(dyadic5.dequant_from_indices(idx5, s)))
    cb = bits.rne_fp16(np.sort(g.uniform(0, 0.1, (n, k // 32, 8)), axis=-1))
    nib = g.integers(0, 16, (n, k)).astype(np.uint8)
    return packing.pack(nib), dict(codebook=dev_f16(cb)), signmag8.dequant_values(cb, nib)


# every m = 1 batched instantiation: the plan's tile height follows the total
# row count (64-row tiles from 1024 tiles up, then 32, then 16), and each
# height is its own kernel, gemv_kernel<CODEC, 64 / height, true, 1, RAGGED>
@pytest.mark.parametrize("codec", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("height,rows", [(64, 65536 + 640), (32, 40000), (16, 3000)])
@pytest.mark.parametrize("k", [128, 256])
def test_gemv_batched_tile_heights(w4, codec, height, rows, k):
    """m = 1 batched GEMV at every tile height for every codec, with k = 128
    (a partial 256-k step: the RAGGED kernels) and k = 256 (whole steps);
    small k keeps the oracle cheap.  The rows are split over 8 problems of
    uneven height."""
    report("gemv_batched_heights", codec=codec, height=height, rows=rows, k=k)
    g = np.random.default_rng(3000 + codec)
    cuts = np.sort(g.choice(np.arange(1, rows), 7, replace=False))
    ns = np.diff(np.concatenate([[0], cuts, [rows]]))
    probs, refs = [], []
    for i, n in enumerate(ns):
        p, side, w_hat = _random_codec_case(codec, int(n), k, 3100 + 10 * codec + i)
        x = synthetic.normal_bf16((1, k), 1.0, 3200 + 10 * codec + i)
        y = torch.full((1, int(n)), float("nan"), device="cuda")
        probs.append(dict(packed=dev_u8(p), x=dev_bf16(x), y=y, **side))
        refs.append((x, w_hat))
    batch = w4.w4_gemv_batched_plan(probs, codec)
    assert batch.info.tile_rows == height and batch.info.flags == (k % 256 != 0)
    batch()
    torch.cuda.synchronize()
    for pr, (x, w_hat) in zip(probs, refs):
        _gemv_check(pr["y"], x, w_hat, False)


def _overflowing_case(codec, n, k, seed):
    """Rows alternate between ordinary side data and side data whose first
    three 64-groups rebuild to +-inf (LUT16 / LUT16S: scale and levels at the
    bf16 maximum; SIGNMAG8: +inf magnitudes).  Returns packed, side tables and
    the fp64 dequantized weight (inf on the overflowing rows)."""
    g = np.random.default_rng(seed)
    idx = g.integers(0, 16, (n, k)).astype(np.uint8)
    if codec in (1, 3):
        s = bits.rne_bf16(g.uniform(0.01, 0.05, (n, k // 64)))
        s[1::2, :3] = 0x7F7F
        L = bits.rne_bf16(np.sort(g.uniform(-1, 1, (n, k // 64, 16)), axis=-1))
        L[1::2, :3, :] = np.where(g.integers(0, 2, (16,)) == 1, 0x7F7F, 0xFF7F)
        if codec == 3:
            T = bits.rne_bf16(np.sort(g.uniform(-1, 1, 16)))
            T[[0, 15]] = [0xFF7F, 0x7F7F]   # s * T overflows for these two
            # the ordinary rows use the same table: scales near 2^-120 keep
            # their weights (at most about 2^8) and their sums well inside fp32
            s[0::2] = bits.rne_bf16(g.uniform(1, 2, s[0::2].shape) * 2.0 ** -120)
            tables = np.ascontiguousarray(np.broadcast_to(T, (n, k // 64, 16)))
            return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(T)),
                    bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables)))
        return (packing.pack(idx), dict(scales=dev_bf16(s), codebook=dev_bf16(L)),
                bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, L)))
    cb = bits.rne_fp16(np.sort(g.uniform(0, 0.1, (n, k // 32, 8)), axis=-1))
    cb[1::2, :6, :] = 0x7C00
    return packing.pack(idx), dict(codebook=dev_f16(cb)), signmag8.dequant_values(cb, idx)


@pytest.mark.parametrize("codec", [1, 2, 3])
@pytest.mark.parametrize("k,m", [(320, 1), (576, 1), (2112, 1), (320, 4), (2112, 7)])
def test_gemv_ragged_k_next_row_overflow(w4, codec, k, m):
    """k not a multiple of 256: the last step of every row has lanes past k,
    which would read the next row's bytes.  Here every other row rebuilds to
    +-inf in its first groups; the finite rows must still match the oracle
    (their padded lanes contribute exact zeros, not inf * 0 = NaN).  Single
    calls (m = 4 and 7 also split k across blocks) and the batched launch."""
    n = 96
    report("gemv_ragged_overflow", codec=codec, k=k, m=m)
    p, side, w_hat = _overflowing_case(codec, n, k, 3300 + k + m + codec)
    x = synthetic.normal_bf16((m, k), 1.0, 3400 + k + m)
    finite = np.all(np.isfinite(w_hat), axis=1)
    assert finite.sum() == n // 2
    y = w4.w4_gemv(dev_u8(p), dev_bf16(x), codec, **side)
    yb = torch.full((m, n), float("nan"), device="cuda")
    batch = w4.w4_gemv_batched_plan([dict(packed=dev_u8(p), x=dev_bf16(x), y=yb, **side)], codec)
    batch()
    torch.cuda.synchronize()
    for out in (y, yb):
        got = host_f32(out)[:, finite]
        y_ref, bound = matmul.gemm_ref(x, w_hat[finite])
        assert matmul.within_tolerance(got, y_ref, bound).all()


@pytest.mark.parametrize("m", [1, 2, 16, 200])
def test_matmul_k_zero_writes_zeros(w4, m):
    """k = 0: y is the empty sum, +0 everywhere (GEMV for m <= 16, GEMM for
    every m, fp32 and bf16)."""
    n = 70
    report("matmul_k0", m=m)
    p = torch.empty((n, 0), dtype=torch.uint8, device="cuda")
    s = torch.empty((n, 0), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    fns = [w4.w4_gemm] + ([w4.w4_gemv] if m <= 16 else [])
    for fn in fns:
        for dt in (torch.float32, torch.bfloat16):
            y = fn(p, x, w4.W4_DYADIC, scales=s, y_dtype=dt)
            torch.cuda.synchronize()
            assert y.shape == (m, n)
            raw = y.view(torch.int16 if dt == torch.bfloat16 else torch.int32).cpu().numpy()
            assert np.all(raw == 0)   # +0 bit patterns


@pytest.mark.parametrize("codec", [0, 3, 5])
@pytest.mark.parametrize("m", [1, 3])
def test_gemv_batched_k_zero_problem(w4, codec, m):
    """A batch holding a k = 0 problem among ordinary ones, planned and
    launched through the C ABI with null side tables and a null x for the
    empty problem (the ABI asks for none at k = 0): its y is +0, the other
    problem's y matches the oracle.  Covers the LUT16S table set-up of the
    pair-table (3) and v_perm (5) decodes, which must not read a table there."""
    import ctypes
    report("gemv_batched_k0", codec=codec, m=m)
    n, k, n0 = 200, 512, 70
    p, side, w_hat = _random_codec_case(3 if codec == 5 else codec, n, k, 3700 + codec)
    x = dev_bf16(synthetic.normal_bf16((m, k), 1.0, 3701))
    y = torch.full((m, n), float("nan"), device="cuda")
    y0 = torch.full((m, n0), float("nan"), device="cuda")
    pk = dev_u8(p)
    arr = (w4.W4Problem * 2)()
    ptr = lambda t: t.data_ptr() if t is not None else None
    arr[0] = w4.W4Problem(pk.data_ptr(), ptr(side.get("scales")), ptr(side.get("codebook")),
                          x.data_ptr(), y.data_ptr(), n, k, 0)
    arr[1] = w4.W4Problem(pk.data_ptr(), None, None, None, y0.data_ptr(), n0, 0, 0)
    info = w4.W4BatchInfo()
    assert w4._lib.w4_gemv_batched_plan(codec, m, w4.W4_F32, arr, 2, ctypes.byref(info)) == 0
    table = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8).to("cuda")
    stream = torch.cuda.current_stream()
    assert w4._lib.w4_gemv_batched(codec, m, w4.W4_F32, ctypes.c_void_p(table.data_ptr()),
                                   ctypes.byref(info), ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert np.all(y0.view(torch.int32).cpu().numpy() == 0)
    y_ref, bound = matmul.gemm_ref(host_bits(x), w_hat)
    assert matmul.within_tolerance(host_f32(y), y_ref, bound).all()


def test_signmag8_k_multiple_of_32_only(w4):
    """SIGNMAG8 quantize and dequant take k a multiple of the group of 32
    (here k = 96, an odd number of groups per row); the matrix calls still
    need k % 64 == 0."""
    n, k = 37, 96
    report("signmag8_k32", n=n, k=k)
    w = synthetic.student_t_bf16((n, k), 5, 0.02, 3500)
    cb = native.signmag8_fit(w)
    p, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    d = w4.w4_unpack_dequant(p, w4.W4_SIGNMAG8, codebook=dev_f16(cb))
    torch.cuda.synchronize()
    nib = native.signmag8_indices(w, cb)
    assert np.array_equal(host_u8(p), packing.pack(nib))
    assert np.array_equal(host_bits(d), signmag8.dequant_from_indices(nib, cb))
    with pytest.raises(w4.W4Error):
        w4.w4_gemv(p, dev_bf16(synthetic.normal_bf16((1, k), 1.0, 3501)), w4.W4_SIGNMAG8,
                   codebook=dev_f16(cb))


# single m = 1 calls on matrices of too few rows for 4-wave blocks take one
# 16-row tile per block of 8 or 16 waves that split k (gemv_kernel<CODEC, 8 or
# 16, false, 4, RAGGED>): (2048, 2048) -> 8 waves, (1024, 4096) -> 16,
# (1000, 2112) -> 8 with a partial last step, (40, 70016) -> 16 with k in
# chunks of the block's LDS
@pytest.mark.parametrize("codec", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("n,k", [(2048, 2048), (1024, 4096), (1000, 2112), (40, 70016)])
def test_gemv_m1_wide_blocks(w4, codec, n, k):
    report("gemv_m1_wide", codec=codec, n=n, k=k)
    p, side, w_hat = _random_codec_case(codec, n, k, 3600 + codec + n)
    x = synthetic.normal_bf16((1, k), 1.0, 3700 + n)
    for dt in (torch.float32, torch.bfloat16):
        y = w4.w4_gemv(dev_u8(p), dev_bf16(x), codec, y_dtype=dt, **side)
        torch.cuda.synchronize()
        _gemv_check(y, x, w_hat, dt == torch.bfloat16)


# ------------------------------------------------------------------ LUT16S variants
@pytest.mark.parametrize("n,k", [(300, 1024), (37, 2048), (5, 256)])
def test_lut16s_interleave_layout(w4, n, k):
    """w4_lut16s_interleave == the oracle's layout function, byte for byte."""
    report("lut16s_interleave", n=n, k=k)
    g = np.random.default_rng(3800 + n)
    p = g.integers(0, 256, (n, k // 2)).astype(np.uint8)
    s = g.integers(0, 1 << 16, (n, k // 64)).astype(np.uint16)
    out = w4.w4_lut16s_interleave(dev_u8(p), dev_bf16(s))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(out), lut16.interleave(p, s))


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("n,k", [(300, 1024), (2048, 2048), (64, 70144)])
def test_lut16s_perm_and_interleaved_gemv(w4, m, n, k):
    """The per-nibble v_perm decode (W4_LUT16S_PERM) and the interleaved layout
    (W4_LUT16S_IL, decoded through the byte -> pair table) beside LUT16S:
    single calls within tolerance of the oracle on the LUT16S weight; the
    LUT16S single call, which decodes per nibble, bit-identical to the PERM
    call; the PERM variant's quantize, dequant and GEMM the LUT16S ones, bit
    for bit."""
    report("lut16s_variants", n=n, k=k, m=m)
    w, s, T, tables, idx = _lut16s_case(n, k, 3900 + n + m)
    w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables))
    x = synthetic.normal_bf16((m, k), 1.0, 3901 + m)
    p = packing.pack(idx)
    pd, sd, td, xd = dev_u8(p), dev_bf16(s), dev_bf16(T), dev_bf16(x)
    y3 = w4.w4_gemv(pd, xd, w4.W4_LUT16S, scales=sd, codebook=td)
    y5 = w4.w4_gemv(pd, xd, w4.W4_LUT16S_PERM, scales=sd, codebook=td)
    il = w4.w4_lut16s_interleave(pd, sd)
    y6 = w4.w4_gemv(il, xd, w4.W4_LUT16S_IL, codebook=td)
    yb = w4.w4_gemv(il, xd, w4.W4_LUT16S_IL, codebook=td, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _gemv_check(y3, x, w_hat, False)
    _gemv_check(y5, x, w_hat, False)
    _gemv_check(y6, x, w_hat, False)
    _gemv_check(yb, x, w_hat, True)
    assert torch.equal(y5, y3)
    if n * k <= 1 << 20:
        q5, _ = w4.w4_quantize_pack(dev_bf16(w), w4.W4_LUT16S_PERM, scales=sd, codebook=td)
        d5 = w4.w4_unpack_dequant(pd, w4.W4_LUT16S_PERM, scales=sd, codebook=td)
        g3 = w4.w4_gemm(pd, dev_bf16(synthetic.normal_bf16((130, k), 1.0, 5)), w4.W4_LUT16S,
                        scales=sd, codebook=td)
        g5 = w4.w4_gemm(pd, dev_bf16(synthetic.normal_bf16((130, k), 1.0, 5)), w4.W4_LUT16S_PERM,
                        scales=sd, codebook=td)
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(q5), p)
        assert np.array_equal(host_bits(d5), lut16.dequant_from_indices(idx, s, tables))
        assert torch.equal(g3, g5)


@pytest.mark.parametrize("codec", [3, 5, 6])
@pytest.mark.parametrize("m", [1, 4, 9])
def test_lut16s_variants_batched(w4, codec, m):
    """LUT16S and both variants through the batched launch: problems of
    several shapes (64-row tiles and, for m = 1 over few rows, 32 / 16-row
    tiles, on which LUT16S decodes per nibble as the PERM variant does)."""
    report("lut16s_variants_batched", codec=codec, m=m)
    probs, refs = [], []
    for i, (n, k) in enumerate([(300, 1024), (129, 2048), (64, 256), (1000, 512)]):
        w, s, T, tables, idx = _lut16s_case(n, k, 4000 + 10 * codec + i)
        w_hat = bits.bf16_to_f64(lut16.dequant_from_indices(idx, s, tables))
        x = synthetic.normal_bf16((m, k), 1.0, 4100 + i)
        pd, sd = dev_u8(packing.pack(idx)), dev_bf16(s)
        y = torch.full((m, n), float("nan"), device="cuda")
        if codec == 6:
            probs.append(dict(packed=w4.w4_lut16s_interleave(pd, sd), codebook=dev_bf16(T),
                              x=dev_bf16(x), y=y))
        else:
            probs.append(dict(packed=pd, scales=sd, codebook=dev_bf16(T), x=dev_bf16(x), y=y))
        refs.append((x, w_hat))
    batch = w4.w4_gemv_batched_plan(probs, codec)
    batch()
    torch.cuda.synchronize()
    for pr, (x, w_hat) in zip(probs, refs):
        _gemv_check(pr["y"], x, w_hat, False)


def test_binding_validation(w4):
    """The Python binding's checks of device tensors (dtype, shape,
    contiguity, side-table shape) raise ValueError before any launch, and a
    well-formed call after them still runs."""
    report("binding_validation")
    n, k = 64, 128
    p = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((n, k // 64), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((2, k), dtype=torch.bfloat16, device="cuda")
    bad = [
        (dict(packed=p.float()), "packed has dtype"),
        (dict(x=x.float()), "x has dtype"),
        (dict(x=torch.zeros((2, k + 64), dtype=torch.bfloat16, device="cuda")), "x must be"),
        (dict(scales=torch.zeros((n, 1), dtype=torch.bfloat16, device="cuda")),
         "scales has shape"),
        (dict(scales=torch.zeros((k // 64, n), dtype=torch.bfloat16, device="cuda").t()),
         "scales must be contiguous"),
        (dict(y=torch.empty((2, n + 1), device="cuda")), "y has shape"),
        (dict(y=torch.empty((2, n), dtype=torch.float16, device="cuda")), "y has dtype"),
    ]
    for over, msg in bad:
        a = dict(packed=p, x=x, scales=s, y=None)
        a.update(over)
        with pytest.raises(ValueError, match=msg):
            w4.w4_gemv(a["packed"], a["x"], w4.W4_DYADIC, scales=a["scales"], y=a["y"])
    y = w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.zeros((2, n), device="cuda"))


def test_binding_current_stream(w4):
    """With no stream given, a call enqueues on torch's current stream (the
    binding reads its handle through a cheaper query): the same handle as
    torch.cuda.current_stream(), also inside a stream context, and a call
    made there is ordered after that stream's earlier work."""
    report("binding_current_stream")
    assert w4._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    n, k = 256, 2048
    w = synthetic.normal_bf16((n, k), 0.02, 5100)
    idx, s = native.dyadic_quantize(w)
    p, sd = dev_u8(packing.pack(idx)), dev_bf16(s)
    with torch.cuda.stream(side):
        assert w4._stream(None) == side.cuda_stream
        xb = synthetic.normal_bf16((1, k), 1.0, 5101)
        x = torch.empty((1, k), dtype=torch.bfloat16, device="cuda")
        x.view(torch.int16).copy_(torch.from_numpy(xb.view(np.int16)))  # on `side`
        y = w4.w4_gemv(p, x, w4.W4_DYADIC, scales=sd)
    side.synchronize()
    _gemv_check(y, xb, bits.bf16_to_f64(native.dyadic_dequant(idx, s)), False)
