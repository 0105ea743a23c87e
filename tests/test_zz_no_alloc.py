"""w4_gemm_noalloc (the GEMM for callers that cannot allocate) against w4_gemm,
through the C ABI: bit-identical outputs on two calls in a row, the second
with a smaller input, each also within the oracle's tolerance; a call whose
workspace exceeds the fixed scratch array is refused before any launch."""

import numpy as np
import pytest
import torch

import synthetic
from oracle import bits, matmul, native, packing
from tests.gpu_util import dev_bf16, dev_u8, host_bits, host_f32, report

pytestmark = pytest.mark.gpu


def _case(n, k, m, seed):
    w = synthetic.normal_bf16((n, k), 0.02, seed)
    idx, s = native.dyadic_quantize(w)
    x = synthetic.normal_bf16((m, k), 1.0, seed + 1)
    return packing.pack(idx), s, x, bits.bf16_to_f64(native.dyadic_dequant(idx, s))


def test_gemm_noalloc_matches_gemm_twice():
    import weight_only_bit_unpack_amd as w4
    # the prefill GEMM (36 MiB of scratch: activations + four k-split
    # partials), then a smaller one (128-row blocks, fewer rows and splits)
    for n, k, m in ((8192, 8192, 256), (300, 1024, 100)):
        report("gemm_noalloc", n=n, k=k, m=m)
        p, s, x, w_hat = _case(n, k, m, 4100 + m)
        pd, sd, xd = dev_u8(p), dev_bf16(s), dev_bf16(x)
        for dt in (torch.float32, torch.bfloat16):
            y_ref = w4.w4_gemm(pd, xd, w4.W4_DYADIC, scales=sd, y_dtype=dt)
            y = torch.full_like(y_ref, float("nan"))
            w4.w4_gemm_noalloc(pd, xd, w4.W4_DYADIC, scales=sd, y=y, y_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               y_ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        rows = np.arange(0, n, max(1, n // 40))
        want, bound = matmul.gemm_ref(x, w_hat[rows])
        got = host_f32(w4.w4_gemm_noalloc(pd, xd, w4.W4_DYADIC, scales=sd))[:, rows]
        assert matmul.within_tolerance(got, want, bound).all()


def test_gemm_noalloc_refuses_oversize():
    import weight_only_bit_unpack_amd as w4
    n, k, m = 256, 8192, 4096     # 64 MiB of packed activations alone
    report("gemm_noalloc_oversize", n=n, k=k, m=m)
    p = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((n, k // 64), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    y = torch.full((m, n), 7.0, device="cuda")
    with pytest.raises(w4.W4Error) as e:
        w4.w4_gemm_noalloc(p, x, w4.W4_DYADIC, scales=s, y=y)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())   # nothing was written
