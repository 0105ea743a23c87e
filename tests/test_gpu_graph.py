"""HIP graph capture of a decode + prefill step built from the library's calls.

Every call only enqueues kernels on the stream it is given; the matrix calls
that need scratch memory take it from a per-stream workspace that exists
after the first call on that stream.  After one eager step on the capture
stream, the batched m = 1 GEMV (the 1B decode stack's three shapes), an m = 4
GEMV (k slices + their reduction) and an m = 256 GEMM (activation re-layout,
split-k partials and their reduction) are captured into one graph.  Each of
several replays, with new activations written between them by ordinary eager
work, must equal the eager calls on the same inputs bit for bit (the kernels
are deterministic), and the first replay is also checked against the fp64
oracle.  The library records no memset into the graph.
"""

import numpy as np
import pytest
import torch

import synthetic
from oracle import bits, native
from tests.gpu_util import host_bits, report
from tests.test_gpu_parity import _gemv_check

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import weight_only_bit_unpack_amd as w4
    report("graph_replay")
    shapes = [(2048, 2048), (5632, 2048), (2048, 5632)]
    mats = []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(7, i, 0))
        p, s = w4.w4_quantize_pack(w, w4.W4_DYADIC)
        mats.append((p, s, n, k, host_bits(w)))
        del w
    x1 = [torch.empty((1, k), dtype=torch.bfloat16, device="cuda") for _, _, _, k, _ in mats]
    y1 = [torch.empty((1, n), device="cuda") for _, _, n, _, _ in mats]
    x4 = torch.empty((4, 2048), dtype=torch.bfloat16, device="cuda")
    y4 = torch.empty((4, 5632), device="cuda")
    xg = torch.empty((256, 2048), dtype=torch.bfloat16, device="cuda")
    yg = torch.empty((256, 2048), device="cuda")
    batch = w4.w4_gemv_batched_plan(
        [{"packed": p, "scales": s, "x": x, "y": y} for (p, s, _, _, _), x, y in zip(mats, x1, y1)],
        w4.W4_DYADIC)
    outs = y1 + [y4, yg]

    def step(stream):
        batch(stream)
        w4.w4_gemv(mats[1][0], x4, w4.W4_DYADIC, scales=mats[1][1], y=y4, stream=stream)
        w4.w4_gemm(mats[0][0], xg, w4.W4_DYADIC, scales=mats[0][1], y=yg, stream=stream)

    def fill(r):
        for i, x in enumerate(x1 + [x4, xg]):
            x.copy_(synthetic.normal_bf16_device(tuple(x.shape), 1.0, synthetic.seed(7, 10 * r + i, 1)))
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()

    cap = torch.cuda.Stream()
    fill(0)
    with torch.cuda.stream(cap):
        step(cap)                       # creates this stream's workspaces
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(cap)
    torch.cuda.synchronize()

    for r in range(1, 4):
        fill(r)
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone() for y in outs]
        if r == 1:
            # replay against the oracle: the stack's first matrix at m = 1, the
            # m = 4 GEMV and the GEMM (the same 2048^2 weight), sampled rows
            for (p, s, n, k, wb), x, y in [(mats[0], x1[0], got[0]), (mats[1], x4, got[3]),
                                           (mats[0], xg[:16], got[4][:16])]:
                idx, sc = native.dyadic_quantize(wb)
                rows = np.arange(0, n, 37)
                w_hat = bits.bf16_to_f64(native.dyadic_dequant(idx[rows], sc[rows]))
                _gemv_check(y[:, rows], host_bits(x), w_hat, False)
        for y in outs:
            y.fill_(float("nan"))
        with torch.cuda.stream(cap):
            step(cap)
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b), r
