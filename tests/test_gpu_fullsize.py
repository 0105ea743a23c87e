"""GPU parity at the workloads' full sizes, in the launch configurations that
bench.py times.

Weights are drawn on the device (seeded, the workloads' distributions) and
quantized by the library; the oracle then checks, on the host:
* packed bytes and scales / dequantized values bit for bit -- on every row of
  the 2048^2 and 8192^2 matrices, on sampled rows (always including the first
  and the last, whose 64-row tile is ragged where n % 64 != 0) elsewhere;
* GEMV / GEMM outputs within |y - y_ref| <= 1e-3 * sum|x w_hat| + 1e-6 of the
  fp64 oracle on the same dequantized weights, for every sampled output,
  computed one row at a time.
Codebooks that the library takes as inputs (LUT16 levels, SIGNMAG8
magnitudes) come from the oracle's fit, or from the library's fit checked
against the oracle's.
"""

import numpy as np
import pytest
import torch

import synthetic
from oracle import bits, dyadic5, lut16, matmul, native, packing, signmag8
from tests.gpu_util import dev_bf16, dev_f16, dev_u8, host_bits, host_f32, host_u8, report

pytestmark = pytest.mark.gpu

ROWS = 24  # sampled rows per matrix


@pytest.fixture(scope="module")
def w4():
    import weight_only_bit_unpack_amd as m
    return m


def _rows(n, seed, count=ROWS):
    g = np.random.default_rng(seed)
    pick = g.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _host_rows(t, rows):
    """Rows of a 16-bit device matrix as uint16 bit patterns."""
    idx = torch.as_tensor(rows, device=t.device)
    return host_bits(t.index_select(0, idx))


def _check_outputs(y, cols, x_bits, w_hat_rows, bf16_out=False):
    """y[:, cols] against the fp64 oracle on the rows' dequantized weights."""
    y_ref, bound = matmul.gemm_ref(x_bits, w_hat_rows)
    got = host_f32(y)[:, cols]
    ok = matmul.within_tolerance(got, y_ref, bound, bf16_out=bf16_out)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError(f"{(~ok).sum()} of {ok.size} outside tolerance, e.g. {bad.tolist()}: "
                             f"got {got[tuple(bad[0])]} want {y_ref[tuple(bad[0])]}")


def _dyadic_rows(w_dev, p_dev, s_dev, rows):
    """Bit-exact check of the library's packed bytes and scales on `rows`;
    returns the oracle's dequantized rows as bf16 bits and as fp64."""
    w_rows = _host_rows(w_dev, rows)
    idx, s = native.dyadic_quantize(w_rows)
    got_p = host_u8(p_dev.index_select(0, torch.as_tensor(rows, device=p_dev.device)))
    assert np.array_equal(_host_rows(s_dev, rows), s)
    assert np.array_equal(got_p, packing.pack(idx))
    deq = native.dyadic_dequant(idx, s)
    return deq, bits.bf16_to_f64(deq)


# ------------------------------------------------------------ 2048 x 2048, m = 1
def test_fullsize_dyadic_2048_gemv(w4):
    """Single 2048^2 weight, N(0, 0.02^2), seed 0; every row and output."""
    n = k = 2048
    report("fullsize_dyadic_2048", n=n, k=k)
    w = synthetic.normal_bf16_device((n, k), 0.02, synthetic.seed(0, 0, 0))
    x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(0, 0, 1))
    p, s = w4.w4_quantize_pack(w, w4.W4_DYADIC)
    y = w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s)
    d = w4.w4_unpack_dequant(p, w4.W4_DYADIC, scales=s)
    torch.cuda.synchronize()
    deq, w_hat = _dyadic_rows(w, p, s, np.arange(n))
    assert np.array_equal(host_bits(d), deq)
    _check_outputs(y, np.arange(n), host_bits(x), w_hat)


# ------------------------------------------------------------ the 1B decode stack
def test_fullsize_decode_stack_batched_gemv(w4):
    """168 matrices (24 blocks x q,k,v,o,gate,up,down), Student-t nu = 4 at
    sigma 0.02, one batched m = 1 launch with fp32 outputs -- the pass
    bench.py times."""
    shapes = synthetic.llama1b_stack_shapes()
    report("fullsize_decode_stack", matrices=len(shapes))
    probs, checks = [], []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0))
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(2, i, 1))
        p, s = w4.w4_quantize_pack(w, w4.W4_DYADIC)
        rows = _rows(n, 7000 + i)
        _, w_hat = _dyadic_rows(w, p, s, rows)
        del w
        y = torch.full((1, n), float("nan"), device="cuda")
        probs.append({"packed": p, "scales": s, "x": x, "y": y})
        checks.append((rows, w_hat))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_DYADIC)
    batch()
    torch.cuda.synchronize()
    for pr, (rows, w_hat) in zip(probs, checks):
        _check_outputs(pr["y"], rows, host_bits(pr["x"]), w_hat)


# ------------------------------------------------------------ the 1B stack as DYADIC5
def test_fullsize_dyadic5_stack_batched(w4):
    """The 168 decode-stack matrices quantized to W4_DYADIC5 with a random
    width of 3, 4 or 5 bits per group (as bench.py draws them): both index
    planes and the scales bit-exact on sampled rows, then the one batched
    m = 1 launch."""
    shapes = synthetic.llama1b_stack_shapes()
    report("fullsize_dyadic5_stack", matrices=len(shapes))
    gen = torch.Generator(device="cuda").manual_seed(synthetic.seed(7, 0, 0))
    probs, checks = [], []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0))
        wd = torch.randint(3, 6, (n, k // 64), dtype=torch.uint8, device="cuda", generator=gen)
        p, msb, s = w4.w4_quantize_dyadic5(w, wd)
        rows = _rows(n, 7900 + i, count=8)
        sel = torch.as_tensor(rows, device="cuda")
        idx5, s_o = dyadic5.quantize(_host_rows(w, rows), host_u8(wd.index_select(0, sel)))
        nib, hi = dyadic5.planes(idx5)
        assert np.array_equal(_host_rows(s, rows), s_o)
        assert np.array_equal(host_u8(p.index_select(0, sel)), nib)
        assert np.array_equal(host_u8(msb.index_select(0, sel)), hi)
        del w, wd
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(2, i, 1))
        y = torch.full((1, n), float("nan"), device="cuda")
        probs.append({"packed": p, "codebook": msb, "scales": s, "x": x, "y": y})
        checks.append((rows, bits.bf16_to_f64(dyadic5.dequant_from_indices(idx5, s_o))))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_DYADIC5)
    batch()
    torch.cuda.synchronize()
    for pr, (rows, w_hat) in zip(probs, checks):
        _check_outputs(pr["y"], rows, host_bits(pr["x"]), w_hat)


# ------------------------------------------------------------ 3.9B-sized LUT16
@pytest.mark.parametrize("n,k", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_fullsize_lut16(w4, n, k):
    """N(0, 0.015^2) with 0.1% outliers at +-10 sigma; k-means fit (quantile
    start, 25 Lloyd rounds) on the GPU, equal to the oracle's on every group;
    quantize, dequant and GEMV at m = 1, 4, 16 on sampled rows."""
    report("fullsize_lut16", n=n, k=k)
    w = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                              synthetic.seed(3, n + k, 0))
    s, L = native.lut16_fit(host_bits(w))
    # the library's own fit is the oracle's, bit for bit, on the whole matrix
    s_dev, L_dev = w4.w4_lut16_fit(w)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(s_dev), s)
    assert np.array_equal(host_bits(L_dev), L)
    p, _ = w4.w4_quantize_pack(w, w4.W4_LUT16, scales=s_dev, codebook=L_dev)
    d = w4.w4_unpack_dequant(p, w4.W4_LUT16, scales=s_dev, codebook=L_dev)
    torch.cuda.synchronize()
    rows = _rows(n, 7300 + n + k)
    sel = torch.as_tensor(rows, device="cuda")
    idx = native.lut16_indices(_host_rows(w, rows), s[rows], L[rows])
    assert np.array_equal(host_u8(p.index_select(0, sel)), packing.pack(idx))
    deq = lut16.dequant_from_indices(idx, s[rows], L[rows])
    assert np.array_equal(host_bits(d.index_select(0, sel)), deq)
    w_hat = bits.bf16_to_f64(deq)
    del w, d
    for m in (1, 4, 16):
        x = synthetic.normal_bf16_device((m, k), 1.0, synthetic.seed(3, n + k, m))
        y = w4.w4_gemv(p, x, w4.W4_LUT16, scales=s_dev, codebook=L_dev)
        torch.cuda.synchronize()
        _check_outputs(y, rows, host_bits(x), w_hat)


# ------------------------------------------------------------ 3.9B-sized LUT16S
def test_fullsize_lut16s_batched():
    """The three 3.9B-sized matrices in the one-table reading (4.25 bits per
    weight): group scales = absmax (oracle, whole matrix), the table from the
    oracle's whole-weight k-means over the first 512 rows of each matrix;
    quantize + dequant bit-exact and one batched m = 1 GEMV over all three on
    sampled rows, for each of the codec's three decodes."""
    import weight_only_bit_unpack_amd as w4
    report("fullsize_lut16s")
    probs, checks = [], []
    for i, (n, k) in enumerate(synthetic.llama39b_shapes()):
        w = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                                  synthetic.seed(6, i, 0))
        wb = host_bits(w)
        s = lut16.group_scales(wb)
        _, T = lut16.fit_shared(wb[:512], iters=10)
        args = dict(scales=dev_bf16(s), codebook=dev_bf16(T))
        p, _ = w4.w4_quantize_pack(w, w4.W4_LUT16S, **args)
        d = w4.w4_unpack_dequant(p, w4.W4_LUT16S, **args)
        torch.cuda.synchronize()
        rows = _rows(n, 8100 + i)
        sel = torch.as_tensor(rows, device="cuda")
        tables = np.ascontiguousarray(lut16.shared_tables(s[rows], T))
        idx = native.lut16_indices(wb[rows], s[rows], tables)
        assert np.array_equal(host_u8(p.index_select(0, sel)), packing.pack(idx))
        deq = lut16.dequant_from_indices(idx, s[rows], tables)
        assert np.array_equal(host_bits(d.index_select(0, sel)), deq)
        del w, d, wb
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(6, i, 1))
        y = torch.full((1, n), float("nan"), device="cuda")
        probs.append(dict(packed=p, x=x, y=y, **args))
        checks.append((rows, bits.bf16_to_f64(deq)))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_LUT16S)
    batch()
    torch.cuda.synchronize()
    for pr, (rows, w_hat) in zip(probs, checks):
        _check_outputs(pr["y"], rows, host_bits(pr["x"]), w_hat)
    # the two other decodes of the same weights, as bench.py times them: the
    # per-nibble v_perm lookups (W4_LUT16S_PERM) on the planar arrays, and the
    # interleaved layout (W4_LUT16S_IL)
    perm = [dict(pr, y=torch.full_like(pr["y"], float("nan"))) for pr in probs]
    il = [dict(packed=w4.w4_lut16s_interleave(pr["packed"], pr["scales"]),
               codebook=pr["codebook"], x=pr["x"], y=torch.full_like(pr["y"], float("nan")))
          for pr in probs]
    w4.w4_gemv_batched_plan(perm, w4.W4_LUT16S_PERM)()
    w4.w4_gemv_batched_plan(il, w4.W4_LUT16S_IL)()
    torch.cuda.synchronize()
    for variant in (perm, il):
        for pr, (rows, w_hat) in zip(variant, checks):
            _check_outputs(pr["y"], rows, host_bits(pr["x"]), w_hat)


# ------------------------------------------------------------ 2B SIGNMAG8, warm start
def test_fullsize_signmag8_warm():
    """The warm-start fit on two whole 2048^2 Student-t (nu = 5) matrices in
    one call each; 1024 sampled groups of each against the oracle."""
    import weight_only_bit_unpack_amd as w4
    from tests.test_gpu_parity import _warm_check
    report("fullsize_signmag8_warm")
    for i in range(2):
        w = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, i, 0))
        cb, pr = w4.w4_signmag8_fit_warm(w)
        torch.cuda.synchronize()
        groups = np.random.default_rng(9100 + i).choice(2048 * 64, 1024, replace=False)
        wb = host_bits(w).reshape(-1, 32)[groups]
        _warm_check(wb, host_bits(cb).reshape(-1, 8)[groups],
                    host_u8(pr).reshape(-1)[groups], 25, max_mismatch=0.01)


# ------------------------------------------------------------ 2B SIGNMAG8
def test_fullsize_signmag8_stack(w4):
    """The 2B model's 224 matrices of 2048^2, Student-t nu = 5 at sigma 0.02,
    group 32 sign + 3-bit magnitude, exactly as bench.py times them: fp16
    codebooks fitted on the GPU (equal to the oracle's fit on every group of
    the first 16 matrices and on the sampled rows of the others), packed
    bytes and dense dequant bit-exact on sampled rows, then the one batched
    m = 1 launch over all 224 (7168 tiles of 64 rows: the plan keeps 64-row
    tiles, so this runs gemv_kernel<SIGNMAG8, 1, true, 1, false>)."""
    n = k = 2048
    count = 224
    report("fullsize_signmag8", matrices=count)
    probs, checks = [], []
    for i in range(count):
        w = synthetic.student_t_bf16_device((n, k), 5, 0.02, synthetic.seed(4, i, 0))
        cb_dev = w4.w4_signmag8_fit(w)
        p, _ = w4.w4_quantize_pack(w, w4.W4_SIGNMAG8, codebook=cb_dev)
        torch.cuda.synchronize()
        rows = _rows(n, 7600 + i, count=24 if i < 16 else 6)
        sel = torch.as_tensor(rows, device="cuda")
        w_rows = _host_rows(w, rows)
        if i < 16:
            cb = native.signmag8_fit(host_bits(w))
            assert np.array_equal(host_bits(cb_dev), cb)
            cb_rows = cb[rows]
        else:
            cb_rows = native.signmag8_fit(w_rows)
            assert np.array_equal(host_bits(cb_dev.index_select(0, sel)), cb_rows)
        nib = native.signmag8_indices(w_rows, cb_rows)
        assert np.array_equal(host_u8(p.index_select(0, sel)), packing.pack(nib))
        if i < 16:
            d = w4.w4_unpack_dequant(p, w4.W4_SIGNMAG8, codebook=cb_dev)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(d.index_select(0, sel)),
                                  signmag8.dequant_from_indices(nib, cb_rows))
            del d
        del w
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(4, i, 1))
        y = torch.full((1, n), float("nan"), device="cuda")
        probs.append({"packed": p, "codebook": cb_dev, "x": x, "y": y})
        checks.append((rows, signmag8.dequant_values(cb_rows, nib)))
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_SIGNMAG8)
    assert batch.info.tile_rows == 64 and batch.info.total_tiles == count * n // 64
    batch()
    torch.cuda.synchronize()
    for pr, (rows, w_hat) in zip(probs, checks):
        _check_outputs(pr["y"], rows, host_bits(pr["x"]), w_hat)


# ------------------------------------------------------------ prefill GEMM
def test_fullsize_gemm_8192(w4):
    """M = 256, K = N = 8192, dyadic N(0, 0.02^2) weights: quantize_pack
    bit-exact on every row, GEMM (pack + split-k kernel + reduction, as
    bench.py times it) on 40 sampled weight rows x all 256 batch rows, fp32
    and bf16 outputs; and the m = 1 GEMV on the same weight (the single-call
    launch of 16-row tiles with k split over 8 waves that bench.py times)."""
    n = k = 8192
    m = 256
    report("fullsize_gemm", m=m, n=n, k=k)
    w = synthetic.normal_bf16_device((n, k), 0.02, synthetic.seed(5, 0, 0))
    x = synthetic.normal_bf16_device((m, k), 1.0, synthetic.seed(5, 0, 1))
    p, s = w4.w4_quantize_pack(w, w4.W4_DYADIC)
    torch.cuda.synchronize()
    idx, s_o = native.dyadic_quantize(host_bits(w))
    assert np.array_equal(host_bits(s), s_o)
    assert np.array_equal(host_u8(p), packing.pack(idx))
    rows = _rows(n, 7900, count=40)
    w_hat = bits.bf16_to_f64(native.dyadic_dequant(idx[rows], s_o[rows]))
    del w, idx
    y = w4.w4_gemm(p, x, w4.W4_DYADIC, scales=s)
    yb = w4.w4_gemm(p, x, w4.W4_DYADIC, scales=s, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check_outputs(y, rows, host_bits(x), w_hat)
    _check_outputs(yb, rows, host_bits(x), w_hat, bf16_out=True)
    xv = x[:1].contiguous()
    yv = w4.w4_gemv(p, xv, w4.W4_DYADIC, scales=s)
    torch.cuda.synchronize()
    _check_outputs(yv, rows, host_bits(xv), w_hat)
