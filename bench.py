#!/usr/bin/env python3
"""Benchmark of the W4 dequant-GEMV / GEMM hot path on one MI355X.

Headline (`value`): W4A16 GEMV at m = 1 over the whole 1B decode stack -- 24
blocks x (q, k, v, o [2048, 2048]; gate, up [5632, 2048]; down [2048, 5632])
= 168 matrices, 1,233,125,376 dyadic 4-bit weights in groups of 64, Student-t
(nu = 4) weights scaled to sigma 0.02, one N(0, 1) bf16 activation vector per
matrix.  One step = one pass over the stack (one batched launch), inputs
resident in HBM.  `value` = algorithmic bytes of the pass (packed nibbles +
bf16 scales + x + fp32 y) / step time, in GB/s.

Also measured in the same run and reported under "rows" (with a plain 1 GiB
device copy as context for what HBM delivers on the box): the same pass as
168 separate w4_gemv calls, quantize_pack and unpack_dequant over the stack,
and the prefill GEMM (M = 256, K = N = 8192, in TFLOP/s) with quantize_pack of
its 8192^2 weight.  The CPU baseline times the oracle (numpy, one thread) on
the first eight decoder blocks of the stack.

    python bench.py [--gpus 1] [--steps 1000] [--warmup 200]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "W4 dequant-GEMV GB/s (% HBM peak) at m=1; W4A16 GEMM TFLOP/s at m=256"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["headline", "gemm", "copy", "fit", "codec"], default=None,
                    help="run one target only (for profiler runs): the batched decode pass, "
                         "the M=256 GEMM, a 1 GiB device copy that calibrates HBM counters, "
                         "the table / magnitude fits, or quantize + dequant of one 8192^2 "
                         "weight for every codec")
    ap.add_argument("--only-headline", action="store_true", help="same as --only headline")
    a = ap.parse_args()
    if a.only_headline:
        a.only = "headline"
    return a


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the GEMV kernel sources, to tie stored counter readings to code."""
    h = hashlib.sha256()
    for f in ("w4_gemv.hip", "w4_device.h"):
        with open(os.path.join(ROOT, "weight_only_bit_unpack_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(name, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def timed(fn, stream, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def time_gemm(w4, synthetic, torch, dev, stream, args):
    """Prefill GEMM, M = 256, K = N = 8192, dyadic weights N(0, 0.02^2): ms per
    call (pack + GEMM + split-k reduction) and TFLOP/s."""
    log("prefill GEMM M=256, K=N=8192")
    W = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), dev)
    X = synthetic.normal_bf16_device((256, 8192), 1.0, synthetic.seed(5, 0, 1), dev)
    P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
    del W
    Y = torch.empty((256, 8192), dtype=torch.float32, device=dev)
    ms_g = timed(lambda: w4.w4_gemm(P, X, w4.W4_DYADIC, scales=S, y=Y, stream=stream),
                 stream, args.steps, args.warmup)
    return ms_g, 2 * 256 * 8192 * 8192 / (ms_g * 1e-3) / 1e12


def shared_table_levels(w):
    """LUT16S side data for timing runs: group absmax scales and one table of
    16 quantiles of the normalised weights (first 512 rows), built with torch
    on the device.  Throughput does not depend on the values."""
    import torch
    n, k = w.shape
    g = w.float().reshape(n, k // 64, 64)
    s = g.abs().amax(dim=-1, keepdim=True)
    u = torch.where(s > 0, g / torch.where(s > 0, s, torch.ones_like(s)), torch.zeros_like(g))
    v = torch.sort(u[:512].reshape(-1)).values
    q = (torch.arange(16, device=w.device) * (v.numel() // 16) + v.numel() // 32)
    return (s.squeeze(-1).to(torch.bfloat16).contiguous(),
            v[q].to(torch.bfloat16).contiguous())


FIT_STEPS = 5  # timed k-means fits per shape (each takes milliseconds)


def other_configs(w4, synthetic, torch, dev, stream, args):
    """Rows for the 2048^2 single GEMV, the 3.9B-sized LUT16 fits and GEMVs and
    the 2B SIGNMAG8 dequant + batched GEMV."""
    rows = {}
    # single 2048^2 DYADIC weight, N(0, 0.02^2), m = 1: one call's latency
    W = synthetic.normal_bf16_device((2048, 2048), 0.02, synthetic.seed(0, 0, 0), dev)
    x = synthetic.normal_bf16_device((1, 2048), 1.0, synthetic.seed(0, 0, 1), dev)
    P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
    y = torch.empty((1, 2048), device=dev)
    ms = timed(lambda: w4.w4_gemv(P, x, w4.W4_DYADIC, scales=S, y=y, stream=stream), stream,
               args.steps, args.warmup)
    b = 2048 * 1024 + 2 * 2048 * 32 + 2 * 2048 + 4 * 2048
    rows["gemv_m1_2048x2048_single_call"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}
    del W, P, S

    # LUT16 on the 3.9B-sized shapes: k-means fit on the GPU, then GEMV at m = 1, 4, 16
    log("LUT16 3.9B-sized fit + GEMVs")
    for i, (n, k) in enumerate([(4096, 4096), (11008, 4096), (4096, 11008)]):
        W = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                                  synthetic.seed(3, i, 0), dev)
        sc = torch.empty((n, k // 64), dtype=torch.bfloat16, device=dev)
        L = torch.empty((n, k // 64, 16), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: w4.w4_lut16_fit(W, 25, scales=sc, codebook=L, stream=stream),
                   stream, FIT_STEPS, 1)
        rows[f"lut16_fit_{n}x{k}"] = {"ms": ms, "Mgroups/s": n * k / 64 / (ms * 1e-3) / 1e6,
                                      "Gweights/s": n * k / (ms * 1e-3) / 1e9}
        P, _ = w4.w4_quantize_pack(W, w4.W4_LUT16, scales=sc, codebook=L)
        del W
        for m in (1, 4, 16):
            x = synthetic.normal_bf16_device((m, k), 1.0, synthetic.seed(3, i, 1), dev)
            y = torch.empty((m, n), device=dev)
            ms = timed(lambda: w4.w4_gemv(P, x, w4.W4_LUT16, scales=sc, codebook=L, y=y,
                                          stream=stream), stream, args.steps, args.warmup)
            b = n * k // 2 + n * (k // 64) * 34 + 2 * m * k + 4 * m * n
            rows[f"lut16_gemv_m{m}_{n}x{k}"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}
        del P, sc, L

    # LUT16S (one table per matrix, 4.25 bits per weight): the three 3.9B-sized
    # matrices in one batched m = 1 launch
    log("LUT16S 3.9B-sized batched GEMV")
    probs, total = [], 0
    for i, (n, k) in enumerate([(4096, 4096), (11008, 4096), (4096, 11008)]):
        W = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                                  synthetic.seed(6, i, 0), dev)
        sc, T = shared_table_levels(W)
        P, _ = w4.w4_quantize_pack(W, w4.W4_LUT16S, scales=sc, codebook=T)
        del W
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(6, i, 1), dev)
        probs.append({"packed": P, "scales": sc, "codebook": T, "x": x,
                      "y": torch.empty((1, n), device=dev)})
        total += n * k // 2 + n * (k // 64) * 2 + 32 + 2 * k + 4 * n
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_LUT16S)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    rows["lut16s_gemv_m1_3.9b_shapes_batched"] = {"ms": ms, "GB/s": total / (ms * 1e-3) / 1e9}
    del probs, batch

    # DYADIC5 (3/4/5-bit groups in one 5-bit index space): the 1B decode stack
    # with widths 3, 4, 5 drawn per group, one batched m = 1 launch, and the
    # quantizer on the 8192^2 prefill weight
    log("DYADIC5 1B stack batched GEMV")
    gen = torch.Generator(device=dev).manual_seed(synthetic.seed(7, 0, 0))
    probs, total = [], 0
    for i, (n, k) in enumerate(synthetic.llama1b_stack_shapes()):
        W = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0), dev)
        wd = torch.randint(3, 6, (n, k // 64), dtype=torch.uint8, device=dev, generator=gen)
        P, M, S = w4.w4_quantize_dyadic5(W, wd)
        del W, wd
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(2, i, 1), dev)
        probs.append({"packed": P, "codebook": M, "scales": S, "x": x,
                      "y": torch.empty((1, n), device=dev)})
        total += n * k // 2 + n * k // 8 + 2 * n * (k // 64) + 2 * k + 4 * n
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_DYADIC5)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    rows["dyadic5_gemv_m1_llama1b_stack_batched"] = {"ms": ms, "GB/s": total / (ms * 1e-3) / 1e9}
    del probs, batch
    W = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), dev)
    wd = torch.randint(3, 6, (8192, 128), dtype=torch.uint8, device=dev, generator=gen)
    P, M, S = w4.w4_quantize_dyadic5(W, wd)
    ms = timed(lambda: w4.w4_quantize_dyadic5(W, wd, packed=P, msb=M, scales=S, stream=stream),
               stream, 20, 3)
    b = 2 * 8192 * 8192 + 8192 * 128 + 8192 * 4096 + 8192 * 1024 + 2 * 8192 * 128
    rows["quantize_dyadic5_8192x8192"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}
    del W, wd, P, M, S

    # SIGNMAG8: 224 x 2048^2, Student-t nu = 5; dense dequant + one batched m = 1 GEMV
    log("SIGNMAG8 2B stack")
    probs, total = [], 0
    for i in range(224):
        W = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, i, 0), dev)
        cb = w4.w4_signmag8_fit(W, 25, stream=stream)
        if i == 0:
            ms = timed(lambda: w4.w4_signmag8_fit(W, 25, codebook=cb, stream=stream), stream,
                       FIT_STEPS, 1)
            rows["signmag8_fit_2048x2048"] = {"ms": ms,
                                              "Mgroups/s": 2048 * 64 / (ms * 1e-3) / 1e6,
                                              "Gweights/s": 2048 * 2048 / (ms * 1e-3) / 1e9}
            ms = timed(lambda: w4.w4_signmag8_fit_warm(W, 25, stream=stream), stream,
                       FIT_STEPS, 1)
            rows["signmag8_fit_warm_2048x2048"] = {"ms": ms,
                                                   "Mgroups/s": 2048 * 64 / (ms * 1e-3) / 1e6}
        P, _ = w4.w4_quantize_pack(W, w4.W4_SIGNMAG8, codebook=cb, stream=stream)
        del W
        x = synthetic.normal_bf16_device((1, 2048), 1.0, synthetic.seed(4, i, 1), dev)
        probs.append({"packed": P, "codebook": cb, "x": x, "y": torch.empty((1, 2048), device=dev)})
        total += 2048 * 1024 + 2048 * 64 * 16 + 2 * 2048 + 4 * 2048
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_SIGNMAG8)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    nominal = 224 * (2048 * 2048 * 4.25 / 8 + 2 * 2048 + 4 * 2048)
    rows["signmag8_gemv_m1_224x2048x2048"] = {
        "ms": ms, "GB/s": total / (ms * 1e-3) / 1e9,
        "GB/s_at_nominal_4.25_bits": nominal / (ms * 1e-3) / 1e9}
    out = torch.empty((2048, 2048), dtype=torch.float16, device=dev)
    p0 = probs[0]
    ms = timed(lambda: w4.w4_unpack_dequant(p0["packed"], w4.W4_SIGNMAG8, codebook=p0["codebook"],
                                            out=out, stream=stream), stream, args.steps, args.warmup)
    b = 2048 * 1024 + 2048 * 64 * 16 + 2 * 2048 * 2048
    rows["signmag8_dequant_2048x2048"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}
    del probs, batch, out
    torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (the library has no "
                                   "multi-GPU path); run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import synthetic
    import weight_only_bit_unpack_amd as w4

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.only == "codec":
        # quantize_pack (DYADIC) and unpack_dequant (every codec) on one
        # 8192 x 8192 weight, N(0, 0.02^2): ms per call, read + write bytes
        n = k = 8192
        W = synthetic.normal_bf16_device((n, k), 0.02, synthetic.seed(5, 0, 0), dev)
        P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
        ms = timed(lambda: w4.w4_quantize_pack(W, w4.W4_DYADIC, packed=P, scales=S,
                                               stream=stream), stream, args.steps, args.warmup)
        b = 2 * n * k + n * k // 2 + n * k // 32
        print(json.dumps({"target": "quantize_dyadic", "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}),
              flush=True)
        sl, L = w4.w4_lut16_fit(W, 1)
        PL, _ = w4.w4_quantize_pack(W, w4.W4_LUT16, scales=sl, codebook=L)
        cb = w4.w4_signmag8_fit(W, 1)
        P8, _ = w4.w4_quantize_pack(W, w4.W4_SIGNMAG8, codebook=cb)
        wd = torch.full((n, k // 64), 4, dtype=torch.uint8, device=dev)
        P5, M5, S5 = w4.w4_quantize_dyadic5(W, wd)
        out = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
        out16 = torch.empty((n, k), dtype=torch.float16, device=dev)
        cases = [("dequant_dyadic", lambda: w4.w4_unpack_dequant(P, w4.W4_DYADIC, scales=S, out=out,
                                                                 stream=stream), n * k // 2 + n * k // 32),
                 ("dequant_lut16", lambda: w4.w4_unpack_dequant(PL, w4.W4_LUT16, scales=sl, codebook=L,
                                                                out=out, stream=stream),
                  n * k // 2 + n * k // 32 + n * k // 2),
                 ("dequant_signmag8", lambda: w4.w4_unpack_dequant(P8, w4.W4_SIGNMAG8, codebook=cb,
                                                                   out=out16, stream=stream), n * k),
                 ("dequant_dyadic5", lambda: w4.w4_unpack_dequant(P5, w4.W4_DYADIC5, scales=S5,
                                                                  codebook=M5, out=out, stream=stream),
                  n * k // 2 + n * k // 8 + n * k // 32)]
        for name, fn, rb in cases:
            ms = timed(fn, stream, args.steps, args.warmup)
            print(json.dumps({"target": name, "ms": ms, "GB/s": (rb + 2 * n * k) / (ms * 1e-3) / 1e9}),
                  flush=True)
        return
    if args.only == "copy":
        # plain device copy of a known size: what FETCH_SIZE / WRITE_SIZE read
        # for it calibrates the counters (bytes per reported KiB)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms_c = timed(lambda: dst.copy_(src), stream, args.steps, args.warmup)
        print(json.dumps({"target": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "ms": ms_c, "GB/s": 2 * (1 << 30) / (ms_c * 1e-3) / 1e9}), flush=True)
        return
    if args.only == "fit":
        for i, (n, k) in enumerate([(4096, 4096), (11008, 4096), (4096, 11008)]):
            W = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                                      synthetic.seed(3, i, 0), dev)
            ms_f = timed(lambda: w4.w4_lut16_fit(W, 25, stream=stream), stream, args.steps,
                         args.warmup)
            print(json.dumps({"target": "lut16_fit", "shape": [n, k], "ms": ms_f,
                              "Mgroups/s": n * k / 64 / (ms_f * 1e-3) / 1e6}), flush=True)
        W = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, 0, 0), dev)
        ms_f = timed(lambda: w4.w4_signmag8_fit(W, 25, stream=stream), stream, args.steps,
                     args.warmup)
        print(json.dumps({"target": "signmag8_fit", "shape": [2048, 2048], "ms": ms_f,
                          "Mgroups/s": 2048 * 64 / (ms_f * 1e-3) / 1e6}), flush=True)
        ms_f = timed(lambda: w4.w4_signmag8_fit_warm(W, 25, stream=stream), stream,
                     min(args.steps, FIT_STEPS), 1)
        print(json.dumps({"target": "signmag8_fit_warm", "shape": [2048, 2048], "ms": ms_f,
                          "Mgroups/s": 2048 * 64 / (ms_f * 1e-3) / 1e6}), flush=True)
        return
    if args.only == "gemm":
        ms_g, tf = time_gemm(w4, synthetic, torch, dev, stream, args)
        print(json.dumps({"target": "gemm", "ms": ms_g, "TFLOP/s": tf}), flush=True)
        return

    # ---------------------------------------------------------- config 2 stack
    shapes = synthetic.llama1b_stack_shapes()
    log(f"generating + quantizing {len(shapes)} matrices on the GPU")
    mats = []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0), dev)
        x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(2, i, 1), dev)
        packed, scales = w4.w4_quantize_pack(w, w4.W4_DYADIC)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        mats.append({"packed": packed, "scales": scales, "x": x, "y": y, "w": w})
    torch.cuda.synchronize()
    n_weights = sum(n * k for n, k in shapes)
    gemv_bytes = sum(n * k // 2 + 2 * n * (k // 64) + 2 * k + 4 * n for n, k in shapes)

    batch = w4.w4_gemv_batched_plan(
        [{k_: m[k_] for k_ in ("packed", "scales", "x", "y")} for m in mats], w4.W4_DYADIC)

    log("timing the batched decode pass")
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    gbs = gemv_bytes / (ms * 1e-3) / 1e9
    rows = {}
    traffic = stored_traffic("gemv_batched_dyadic_m1_llama1b_stack", gemv_bytes)

    if args.only is None:
        # the same pass as 168 separate calls
        def per_call():
            for m in mats:
                w4.w4_gemv(m["packed"], m["x"], w4.W4_DYADIC, scales=m["scales"], y=m["y"],
                           stream=stream)
        ms_pc = timed(per_call, stream, max(3, args.steps // 4), 2)
        rows["gemv_m1_stack_per_call"] = {"ms": ms_pc, "GB/s": gemv_bytes / (ms_pc * 1e-3) / 1e9,
                                          "launches": len(shapes)}

        # the same 168 launches captured once into a HIP graph and replayed
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            for m in mats:
                w4.w4_gemv(m["packed"], m["x"], w4.W4_DYADIC, scales=m["scales"], y=m["y"],
                           stream=cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for m in mats:
                w4.w4_gemv(m["packed"], m["x"], w4.W4_DYADIC, scales=m["scales"], y=m["y"],
                           stream=cap)
        ms_g = timed(graph.replay, stream, max(3, args.steps // 4), 2)
        rows["gemv_m1_stack_per_call_graph"] = {"ms": ms_g,
                                                "GB/s": gemv_bytes / (ms_g * 1e-3) / 1e9,
                                                "launches": len(shapes)}
        del graph

        # quantize_pack and unpack_dequant over the stack
        q_bytes = sum(2 * n * k + n * k // 2 + 2 * n * (k // 64) for n, k in shapes)

        def quant():
            for m in mats:
                w4.w4_quantize_pack(m["w"], w4.W4_DYADIC, packed=m["packed"], scales=m["scales"],
                                    stream=stream)
        ms_q = timed(quant, stream, 3, 1)
        rows["quantize_pack_stack"] = {"ms": ms_q, "GB/s": q_bytes / (ms_q * 1e-3) / 1e9}

        outs = [torch.empty((n, k), dtype=torch.bfloat16, device=dev) for n, k in shapes[:7]]
        d_bytes = sum(n * k // 2 + 2 * n * (k // 64) + 2 * n * k for n, k in shapes[:7])

        def deq():
            for m, o in zip(mats[:7], outs):
                w4.w4_unpack_dequant(m["packed"], w4.W4_DYADIC, scales=m["scales"], out=o,
                                     stream=stream)
        ms_d = timed(deq, stream, 10, 2)
        rows["unpack_dequant_block"] = {"ms": ms_d, "GB/s": d_bytes / (ms_d * 1e-3) / 1e9,
                                        "matrices": 7}
        del outs

    for m in mats:
        del m["w"]
    torch.cuda.empty_cache()

    if args.only is None:
        # ------------------------------------------------------ config 5 GEMM
        ms_g, tf = time_gemm(w4, synthetic, torch, dev, stream, args)
        rows["gemm_m256_k8192_n8192"] = {"ms": ms_g, "TFLOP/s": tf,
                                         "frac_of_bf16_peak": tf / BF16_MFMA_PEAK_TFLOPS}
        W = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), dev)
        X = synthetic.normal_bf16_device((256, 8192), 1.0, synthetic.seed(5, 0, 1), dev)
        P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
        Y = torch.empty((256, 8192), dtype=torch.float32, device=dev)
        ms_q5 = timed(lambda: w4.w4_quantize_pack(W, w4.W4_DYADIC, packed=P, scales=S,
                                                  stream=stream), stream, 10, 2)
        qb = 2 * 8192 * 8192 + 8192 * 4096 + 2 * 8192 * 128
        rows["quantize_pack_8192x8192"] = {"ms": ms_q5, "GB/s": qb / (ms_q5 * 1e-3) / 1e9}
        # the same weight at other batch sizes (M = 128 takes the 128-row block)
        for mx in (128, 512, 1024):
            Xm = synthetic.normal_bf16_device((mx, 8192), 1.0, synthetic.seed(5, 0, 2), dev)
            Ym = torch.empty((mx, 8192), dtype=torch.float32, device=dev)
            ms_m = timed(lambda: w4.w4_gemm(P, Xm, w4.W4_DYADIC, scales=S, y=Ym, stream=stream),
                         stream, 30, 5)
            tfm = 2 * mx * 8192 * 8192 / (ms_m * 1e-3) / 1e12
            rows[f"gemm_m{mx}_k8192_n8192"] = {"ms": ms_m, "TFLOP/s": tfm,
                                               "frac_of_bf16_peak": tfm / BF16_MFMA_PEAK_TFLOPS}
            del Xm, Ym
        xv = torch.empty((1, 8192), dtype=torch.bfloat16, device=dev).copy_(X[:1])
        yv = torch.empty((1, 8192), dtype=torch.float32, device=dev)
        ms_v5 = timed(lambda: w4.w4_gemv(P, xv, w4.W4_DYADIC, scales=S, y=yv, stream=stream),
                      stream, args.steps, args.warmup)
        vb = 8192 * 4096 + 2 * 8192 * 128 + 2 * 8192 + 4 * 8192
        rows["gemv_m1_8192x8192"] = {"ms": ms_v5, "GB/s": vb / (ms_v5 * 1e-3) / 1e9}
        del W, X, P, S, Y

    if args.only is None:
        rows.update(other_configs(w4, synthetic, torch, dev, stream, args))
        # context: what a plain device copy reaches on this GPU (read + write)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms_c = timed(lambda: dst.copy_(src), stream, 20, 5)
        rows["context_device_copy_1gib"] = {"ms": ms_c,
                                            "GB/s_read_plus_write": 2 * (1 << 30) / (ms_c * 1e-3) / 1e9}
        del src, dst

    # ---------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(mats, shapes)

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama1b_decode_stack_w4a16_gemv_m1", "matrices": len(shapes),
                   "weights": n_weights, "m": 1, "codec": "dyadic", "group": 64,
                   "weight_dist": "student_t_nu4_sigma0.02", "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


CPU_BLOCKS = 8  # decoder blocks of the stack timed on the CPU (about 10-15 s of work)


def cpu_baseline(mats, shapes):
    """The oracle (numpy dequant + fp64 GEMV, one thread) on the first
    CPU_BLOCKS decoder blocks of the stack.  Each weight is regenerated on the
    device, copied to the host and quantized by the oracle's own C routine
    (untimed); the timed part is the oracle's dequant + matmul per matrix."""
    import numpy as np
    import torch
    import synthetic
    from threadpoolctl import threadpool_limits
    from oracle import dyadic, matmul, native, packing
    from oracle.bits import bf16_to_f64

    sample = list(range(7 * CPU_BLOCKS))
    log(f"cpu baseline: oracle on {len(sample)} matrices")
    nbytes, weights, dt = 0, 0, 0.0
    for i in sample:
        n, k = shapes[i]
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0), "cuda")
        wb = w.view(torch.int16).cpu().numpy().view(np.uint16)
        del w
        xb = mats[i]["x"].view(torch.int16).cpu().numpy().view(np.uint16)
        idx, s = native.dyadic_quantize(wb)
        p = packing.pack(idx)
        del wb, idx
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            matmul.gemm_ref(xb, bf16_to_f64(dyadic.dequant(p, s)))
            dt += time.perf_counter() - t0
        nbytes += n * k // 2 + 2 * n * (k // 64) + 2 * k + 4 * n
        weights += n * k
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {CPU_BLOCKS} decoder blocks of the stack ({len(sample)} matrices, "
                      f"{weights:,} weights): numpy dequant + fp64 GEMV, one thread",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
