"""fp64 reference for the fused dequant-GEMV / GEMM, and its error bound.

Oracle (test infrastructure).  The k-means page (section 4.1) routes a
linear layer by batch size m: a LUT kernel for m up to 16, a mixed
4-bit kernel up to 256, plain bf16 GEMM above; the DyadicGumbel page
(section 2.5) unpacks to bf16 and then multiplies.  Either way the result is
``y[i, n] = sum_k x[i, k] * w_hat[n, k]`` on the dequantized weights.

The reference accumulates in fp64 from the same dequantized values the GPU
uses; the bound is ``B[i, n] = sum_k |x[i, k] * w_hat[n, k]|`` and a GPU result
passes when ``|y - y_ref| <= 1e-3 * B + 1e-6``; a bf16 output adds the one
rounding of the output, ``2**-8 * |y_ref|``.  Why any fp32 summation order
passes: a product of a bf16 and a bf16 (or fp16) value is exact in fp32, and
recursive fp32 summation of K terms errs by at most ``K * 2**-24 * B``, below
``1e-3 * B`` for K <= 16760.  Longer sums stay inside the bound when they are
added as blocks of products (dot products of 16 or 32 terms, then the block
sums): about ``(K / 16 + 16) * 2**-24 * B``.
"""

import numpy as np

from .bits import bf16_to_f64

REL_TOL = 1e-3
ABS_TOL = 1e-6
BF16_OUT_REL = 2.0 ** -8


def gemm_ref(x_bits, w_hat):
    """x bf16 bits [M, K], w_hat fp64 [N, K] -> (y fp64 [M, N], bound fp64 [M, N])."""
    x = bf16_to_f64(x_bits)
    w = np.asarray(w_hat, dtype=np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def within_tolerance(y, y_ref, bound, bf16_out=False):
    """Element-wise pass/fail of a GPU result against the fp64 reference."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    tol = REL_TOL * np.asarray(bound, dtype=np.float64) + ABS_TOL
    if bf16_out:
        tol = tol + BF16_OUT_REL * np.abs(y_ref)
    return np.abs(y - y_ref) <= tol
