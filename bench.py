#!/usr/bin/env python3
"""Benchmark of the W4 dequant-GEMV / GEMM hot path on one MI355X.

Headline (`value`): W4A16 GEMV at m = 1 over the whole 1B decode stack -- 24
blocks x (q, k, v, o [2048, 2048]; gate, up [5632, 2048]; down [2048, 5632])
= 168 matrices, 1,233,125,376 dyadic 4-bit weights in groups of 64, Student-t
(nu = 4) weights scaled to sigma 0.02, one N(0, 1) bf16 activation vector per
matrix.  One step = one pass over the stack (one batched launch), inputs
resident in HBM.  `value` = algorithmic bytes of the pass (packed nibbles +
bf16 scales + x + fp32 y) / step time, in GB/s.

Also measured in the same run and reported under "rows": the same pass as
168 separate w4_gemv calls, quantize_pack and unpack_dequant, the prefill GEMM
(M = 256, K = N = 8192, in TFLOP/s) with quantize_pack of its 8192^2 weight,
and the other workloads' rows.  Single calls are timed both by a Python launch
loop and as replays of a HIP graph of many such calls, and the faster counts
(from Python a small call is bound by the binding's per-call checks on the
host; one row gives that rate); single GEMV calls are also
timed rotating over copies of the weight that together exceed the 256 MB
Infinity Cache (rows ending in "_rotating"), so that each call reads HBM.
"context" holds what this GPU delivers in the
same run: a plain streaming read of 4 GiB with 16-byte loads (the read
ceiling the GEMV is set against), the end-to-end time of one such read over
2.25 MiB (the floor under a single small call), a 1 GiB device copy, and the
vendor library's dense bf16 GEMM (torch linear on an unquantized weight) at
the prefill GEMM's shape.  The CPU baseline
times the C oracle (OpenMP on the host's cores) on the whole decode stack,
with further rows for the other workloads, each with its GPU:CPU ratio.

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
    ap.add_argument("--only", choices=["headline", "gemm", "copy", "fit", "codec", "singles",
                                       "lut16s", "variants", "floors"],
                    default=None,
                    help="run one target only (for profiler runs): the batched decode pass, "
                         "the M=256 GEMM, a 1 GiB device copy that calibrates HBM counters, "
                         "the table / magnitude fits, quantize + dequant of one 8192^2 "
                         "weight for every codec, single m = 1 GEMV calls (DYADIC 8192^2, "
                         "LUT16 on the 3.9B shapes), the decode stack as LUT16S in its three "
                         "decode variants, or the batched m = 1 passes of the other codecs "
                         "(DYADIC5 decode stack, 224-matrix SIGNMAG8 stack, the 3.9B-sized "
                         "matrices as LUT16S in its three decode variants), or what single "
                         "calls can reach: a plain read of 2.4 MB and of 37.7 MB per call "
                         "(one buffer, and rotating over 16) beside the 8192^2 DYADIC GEMV, "
                         "each by a launch loop and by graph replays")
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


INFINITY_CACHE_BYTES = 256 << 20  # the MI355X's last-level (MALL) cache


def rotation_copies(weight_bytes):
    """Copies of a weight whose bytes together exceed twice the Infinity
    Cache, so that rotating over them makes every call read from HBM."""
    return max(2, -(-2 * INFINITY_CACHE_BYTES // weight_bytes))


def timed_single(calls, stream, steps, warmup):
    """ms per call of back-to-back single library calls (`calls`, each taking
    the stream to enqueue on, round robin), and how it was timed: the faster
    of a Python launch loop and replays of a HIP graph of the same calls.
    From Python, a small call is bound by the host (the binding's argument
    checks take longer than a 2048^2 GEMV's kernel); a graph removes that
    cost but adds a little per node (0.8 us on the 8192^2 GEMV on one
    machine), so each method wins somewhere."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)](stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        calls[i % len(calls)](stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_loop = e0.elapsed_time(e1) / steps
    ms_graph = timed_calls(calls, stream, steps, warmup)
    return (ms_graph, "graph") if ms_graph < ms_loop else (ms_loop, "python_loop")


def timed_calls(calls, stream, steps, warmup, per_graph=32):
    """ms per call of single library calls on the GPU: `calls` (each takes
    the stream to enqueue on), round robin, at least per_graph of them
    captured into one HIP graph whose replays are timed."""
    import torch
    seq = [calls[i % len(calls)] for i in range(max(per_graph, len(calls)))]
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        for f in seq:  # eagerly first: a call's workspace is made outside the capture
            f(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for f in seq:
            f(cap)
    ms = timed(graph.replay, stream, max(2, steps // len(seq)), max(1, warmup // len(seq)))
    del graph
    return ms / len(seq)


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


def read_ceiling(torch, dev, stream):
    """GB/s of a plain streaming read of 4 GiB with 16-byte nontemporal loads
    (libw4ctx.so), best of a few grid sizes: the read rate HBM delivers to a
    read-only kernel on this GPU; and ms per call of the same kernel over
    2.25 MiB, back to back, timed as the single GEMV calls are."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_bit_unpack_amd", "libw4ctx.so"))
    lib.w4ctx_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
    lib.w4ctx_read_stream.restype = ctypes.c_int
    nbytes = 4 << 30
    buf = torch.full((nbytes // 4,), 0x01010101, dtype=torch.int32, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    best = 0.0
    for blocks in (8192, 16384, 32768):
        def run():
            rc = lib.w4ctx_read_stream(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                       ctypes.c_void_p(sink.data_ptr()), blocks,
                                       ctypes.c_void_p(stream.cuda_stream))
            assert rc == 0, rc
        ms = timed(run, stream, 20, 3)
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    # one call of the same kernel over 2.25 MiB (the 2048^2 weight's size):
    # the time a launch of a small streaming kernel takes end to end
    small = 9 << 18
    buf2 = torch.full((small // 4,), 0x01010101, dtype=torch.int32, device=dev)

    def run_small(st):
        rc = lib.w4ctx_read_stream(ctypes.c_void_p(buf2.data_ptr()), small,
                                   ctypes.c_void_p(sink.data_ptr()), 1024,
                                   ctypes.c_void_p(st.cuda_stream))
        assert rc == 0, rc
    ms_small, _ = timed_single([run_small], stream, 320, 32)  # as single GEMV calls are timed
    del buf, buf2, sink
    torch.cuda.empty_cache()
    return best, ms_small


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


def lut16s_shapes_problems(w4, synthetic, torch, dev):
    """The three 3.9B-sized matrices as LUT16S (N(0, 0.015^2) + outliers, a
    table of 16 quantiles per matrix), one m = 1 problem each; returns the
    problems and their algorithmic bytes."""
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
    return probs, total


def dyadic5_stack_problems(w4, synthetic, torch, dev, gen):
    """The 1B decode stack as DYADIC5 with widths 3, 4, 5 drawn per group
    from gen, one m = 1 problem per matrix; problems and algorithmic bytes."""
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
    return probs, total


def signmag8_stack_problems(w4, synthetic, torch, dev, stream):
    """The 2B model's 224 [2048, 2048] matrices (Student-t nu = 5) as SIGNMAG8
    with magnitudes fitted on the GPU, one m = 1 problem each; problems and
    algorithmic (actual) bytes."""
    probs, total = [], 0
    for i in range(224):
        W = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, i, 0), dev)
        cb = w4.w4_signmag8_fit(W, 25, stream=stream)
        P, _ = w4.w4_quantize_pack(W, w4.W4_SIGNMAG8, codebook=cb, stream=stream)
        del W
        x = synthetic.normal_bf16_device((1, 2048), 1.0, synthetic.seed(4, i, 1), dev)
        probs.append({"packed": P, "codebook": cb, "x": x, "y": torch.empty((1, 2048), device=dev)})
        total += 2048 * 1024 + 2048 * 64 * 16 + 2 * 2048 + 4 * 2048
    return probs, total


def other_configs(w4, synthetic, torch, dev, stream, args):
    """Rows for the 2048^2 single GEMV, the 3.9B-sized LUT16 fits and GEMVs and
    the 2B SIGNMAG8 dequant + batched GEMV."""
    rows = {}
    # single 2048^2 DYADIC weight, N(0, 0.02^2), m = 1: one call's latency
    W = synthetic.normal_bf16_device((2048, 2048), 0.02, synthetic.seed(0, 0, 0), dev)
    x = synthetic.normal_bf16_device((1, 2048), 1.0, synthetic.seed(0, 0, 1), dev)
    P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
    y = torch.empty((1, 2048), device=dev)
    b = 2048 * 1024 + 2 * 2048 * 32 + 2 * 2048 + 4 * 2048
    ms, how = timed_single([lambda st: w4.w4_gemv(P, x, w4.W4_DYADIC, scales=S, y=y, stream=st)],
                           stream, args.steps, args.warmup)
    rows["gemv_m1_2048x2048_single_call"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                             "timing": how}
    # the same call issued one by one from Python: the binding's per-call
    # host cost, not the GPU, sets this rate
    ms = timed(lambda: w4.w4_gemv(P, x, w4.W4_DYADIC, scales=S, y=y, stream=stream), stream,
               args.steps, args.warmup)
    rows["gemv_m1_2048x2048_python_call"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}
    # the same call rotating over 256 copies of the weight (about 600 MB, more
    # than the 256 MB Infinity Cache holds), so each call reads its weight
    # from HBM rather than from a cache that the previous call warmed
    pool = [(P.clone(), S.clone()) for _ in range(256)]
    calls = [lambda st, p=p, s=s: w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s, y=y, stream=st)
             for p, s in pool]
    ms, how = timed_single(calls, stream, max(args.steps, 256), min(args.warmup, 256))
    rows["gemv_m1_2048x2048_rotating_256"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                              "copies": len(pool), "timing": how}
    del W, P, S, pool, calls

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
        wb = n * k // 2 + n * (k // 64) * 34
        pool = [(P.clone(), sc.clone(), L.clone()) for _ in range(rotation_copies(wb))]
        for m in (1, 4, 16):
            x = synthetic.normal_bf16_device((m, k), 1.0, synthetic.seed(3, i, 1), dev)
            y = torch.empty((m, n), device=dev)
            ms, how = timed_single([lambda st: w4.w4_gemv(P, x, w4.W4_LUT16, scales=sc,
                                                          codebook=L, y=y, stream=st)],
                                   stream, args.steps, args.warmup)
            b = wb + 2 * m * k + 4 * m * n
            rows[f"lut16_gemv_m{m}_{n}x{k}"] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                                                "timing": how}
            # the same call over copies of the weight totalling more than the
            # Infinity Cache holds, so each call reads its weight from HBM
            calls = [lambda st, p=p, s=s, c=c: w4.w4_gemv(p, x, w4.W4_LUT16, scales=s,
                                                          codebook=c, y=y, stream=st)
                     for p, s, c in pool]
            ms, how = timed_single(calls, stream, max(args.steps, 4 * len(pool)), args.warmup)
            rows[f"lut16_gemv_m{m}_{n}x{k}_rotating"] = {
                "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9, "copies": len(pool), "timing": how}
        del P, sc, L, pool

    # LUT16S (one table per matrix, 4.25 bits per weight): the three 3.9B-sized
    # matrices in one batched m = 1 launch
    log("LUT16S 3.9B-sized batched GEMV")
    probs, total = lut16s_shapes_problems(w4, synthetic, torch, dev)
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_LUT16S)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    rows["lut16s_gemv_m1_3.9b_shapes_batched"] = {"ms": ms, "GB/s": total / (ms * 1e-3) / 1e9}
    # the same three matrices decoded by per-nibble v_perm lookups instead of
    # the byte -> pair table, and with the scales interleaved into the packed
    # rows (same algorithmic bytes)
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_LUT16S_PERM)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    rows["lut16s_perm_gemv_m1_3.9b_shapes_batched"] = {"ms": ms,
                                                       "GB/s": total / (ms * 1e-3) / 1e9}
    il = [dict(packed=w4.w4_lut16s_interleave(p["packed"], p["scales"]), codebook=p["codebook"],
               x=p["x"], y=p["y"]) for p in probs]
    batch = w4.w4_gemv_batched_plan(il, w4.W4_LUT16S_IL)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    rows["lut16s_il_gemv_m1_3.9b_shapes_batched"] = {"ms": ms, "GB/s": total / (ms * 1e-3) / 1e9}
    del probs, batch, il

    # DYADIC5 (3/4/5-bit groups in one 5-bit index space): the 1B decode stack
    # with widths 3, 4, 5 drawn per group, one batched m = 1 launch, and the
    # quantizer on the 8192^2 prefill weight
    log("DYADIC5 1B stack batched GEMV")
    gen = torch.Generator(device=dev).manual_seed(synthetic.seed(7, 0, 0))
    probs, total = dyadic5_stack_problems(w4, synthetic, torch, dev, gen)
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
    W = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, 0, 0), dev)
    cb = w4.w4_signmag8_fit(W, 25, stream=stream)
    ms = timed(lambda: w4.w4_signmag8_fit(W, 25, codebook=cb, stream=stream), stream,
               FIT_STEPS, 1)
    rows["signmag8_fit_2048x2048"] = {"ms": ms, "Mgroups/s": 2048 * 64 / (ms * 1e-3) / 1e6,
                                      "Gweights/s": 2048 * 2048 / (ms * 1e-3) / 1e9}
    ms = timed(lambda: w4.w4_signmag8_fit_warm(W, 25, stream=stream), stream, FIT_STEPS, 1)
    rows["signmag8_fit_warm_2048x2048"] = {"ms": ms, "Mgroups/s": 2048 * 64 / (ms * 1e-3) / 1e6}
    del W, cb
    probs, total = signmag8_stack_problems(w4, synthetic, torch, dev, stream)
    batch = w4.w4_gemv_batched_plan(probs, w4.W4_SIGNMAG8)
    ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
    nominal = 224 * (2048 * 2048 * 4.25 / 8 + 2 * 2048 + 4 * 2048)
    rows["signmag8_gemv_m1_224x2048x2048"] = {
        "ms": ms, "GB/s": total / (ms * 1e-3) / 1e9,
        "GB/s_at_nominal_4.25_bits": nominal / (ms * 1e-3) / 1e9}
    out = torch.empty((2048, 2048), dtype=torch.float16, device=dev)
    p0 = probs[0]
    ms = timed_single([lambda st: w4.w4_unpack_dequant(p0["packed"], w4.W4_SIGNMAG8,
                                                       codebook=p0["codebook"], out=out, stream=st)],
                      stream, args.steps, args.warmup)[0]
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
        # quantize against the fitted tables / magnitudes (exact nearest level)
        for name, fn in (("quantize_lut16", lambda: w4.w4_quantize_pack(
                              W, w4.W4_LUT16, scales=sl, codebook=L, packed=PL, stream=stream)),
                         ("quantize_signmag8", lambda: w4.w4_quantize_pack(
                              W, w4.W4_SIGNMAG8, codebook=cb, packed=P8, stream=stream))):
            ms = timed(fn, stream, args.steps, args.warmup)
            print(json.dumps({"target": name, "ms": ms, "GB/s": (2 * n * k + n * k // 2) /
                              (ms * 1e-3) / 1e9}), flush=True)
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
    if args.only == "lut16s":
        # the 1B decode stack as LUT16S (one table of 16 quantiles per matrix),
        # one batched m = 1 launch per decode variant: byte -> pair table
        # (LUT16S), per-nibble v_perm lookups (LUT16S_PERM), scales interleaved
        # into the packed rows (LUT16S_IL)
        probs, total = [], 0
        for i, (n, k) in enumerate(synthetic.llama1b_stack_shapes()):
            W = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0), dev)
            sc, T = shared_table_levels(W)
            P, _ = w4.w4_quantize_pack(W, w4.W4_LUT16S, scales=sc, codebook=T)
            del W
            x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(2, i, 1), dev)
            probs.append({"packed": P, "scales": sc, "codebook": T, "x": x,
                          "y": torch.empty((1, n), device=dev)})
            total += n * k // 2 + 2 * n * (k // 64) + 32 + 2 * k + 4 * n
        il = [dict(packed=w4.w4_lut16s_interleave(p["packed"], p["scales"]),
                   codebook=p["codebook"], x=p["x"], y=p["y"]) for p in probs]
        for name, codec, pr in (("lut16s", w4.W4_LUT16S, probs),
                                ("lut16s_perm", w4.W4_LUT16S_PERM, probs),
                                ("lut16s_il", w4.W4_LUT16S_IL, il)):
            batch = w4.w4_gemv_batched_plan(pr, codec)
            ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
            print(json.dumps({"target": f"{name}_gemv_m1_llama1b_stack", "ms": ms,
                              "GB/s": total / (ms * 1e-3) / 1e9}), flush=True)
        return
    if args.only == "variants":
        gen = torch.Generator(device=dev).manual_seed(synthetic.seed(7, 0, 0))
        probs, total = dyadic5_stack_problems(w4, synthetic, torch, dev, gen)
        cases = [("dyadic5_gemv_m1_llama1b_stack", w4.W4_DYADIC5, probs, total)]
        probs, total = signmag8_stack_problems(w4, synthetic, torch, dev, stream)
        cases.append(("signmag8_gemv_m1_224x2048x2048", w4.W4_SIGNMAG8, probs, total))
        probs, total = lut16s_shapes_problems(w4, synthetic, torch, dev)
        il = [dict(packed=w4.w4_lut16s_interleave(p["packed"], p["scales"]),
                   codebook=p["codebook"], x=p["x"], y=p["y"]) for p in probs]
        cases += [("lut16s_gemv_m1_3.9b_shapes", w4.W4_LUT16S, probs, total),
                  ("lut16s_perm_gemv_m1_3.9b_shapes", w4.W4_LUT16S_PERM, probs, total),
                  ("lut16s_il_gemv_m1_3.9b_shapes", w4.W4_LUT16S_IL, il, total)]
        for name, codec, pr, b in cases:
            batch = w4.w4_gemv_batched_plan(pr, codec)
            ms = timed(lambda: batch(stream), stream, args.steps, args.warmup)
            print(json.dumps({"target": name, "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9}),
                  flush=True)
        return
    if args.only == "floors":
        import ctypes
        lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_bit_unpack_amd", "libw4ctx.so"))
        lib.w4ctx_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)

        def both(calls):  # us per call: launch loop, graph replays
            t0 = timed(lambda: [c(stream) for c in calls], stream, max(1, args.steps // len(calls)),
                       max(1, args.warmup // len(calls))) / len(calls)
            return t0 * 1e3, timed_calls(calls, stream, args.steps, args.warmup) * 1e3
        for nbytes, copies in ((9 << 18, 1), (36 << 20, 1), (36 << 20, 16)):
            bufs = [torch.full((nbytes // 4,), 0x01010101, dtype=torch.int32, device=dev)
                    for _ in range(copies)]
            for blocks in (256, 1024, 4096):
                calls = [lambda st, b=b: lib.w4ctx_read_stream(
                    b.data_ptr(), nbytes, sink.data_ptr(), blocks, st.cuda_stream) for b in bufs]
                us_loop, us_graph = both(calls)
                print(json.dumps({"target": "read", "bytes": nbytes, "copies": copies,
                                  "blocks": blocks, "us_loop": us_loop, "us_graph": us_graph}),
                      flush=True)
            del bufs
        W = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), dev)
        P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
        del W
        x = synthetic.normal_bf16_device((1, 8192), 1.0, synthetic.seed(5, 0, 1), dev)
        y = torch.empty((1, 8192), device=dev)
        for copies in (1, 16):
            pool = [(P, S)] + [(P.clone(), S.clone()) for _ in range(copies - 1)]
            calls = [lambda st, p=p, s=s: w4.w4_gemv(p, x, w4.W4_DYADIC, scales=s, y=y, stream=st)
                     for p, s in pool]
            us_loop, us_graph = both(calls)
            print(json.dumps({"target": "gemv_m1_8192x8192", "copies": copies,
                              "us_loop": us_loop, "us_graph": us_graph}), flush=True)
        return
    if args.only == "singles":
        W = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), dev)
        P, S = w4.w4_quantize_pack(W, w4.W4_DYADIC)
        x = synthetic.normal_bf16_device((1, 8192), 1.0, synthetic.seed(5, 0, 1), dev)
        y = torch.empty((1, 8192), device=dev)
        ms, how = timed_single([lambda st: w4.w4_gemv(P, x, w4.W4_DYADIC, scales=S, y=y,
                                                      stream=st)], stream, args.steps, args.warmup)
        b = 8192 * 4096 + 2 * 8192 * 128 + 2 * 8192 + 4 * 8192
        print(json.dumps({"target": "gemv_m1_8192x8192", "ms": ms, "GB/s": b / (ms * 1e-3) / 1e9,
                          "timing": how}), flush=True)
        del W, P, S
        for i, (n, k) in enumerate([(4096, 4096), (11008, 4096), (4096, 11008)]):
            W = synthetic.normal_outliers_bf16_device((n, k), 0.015, 0.001, 0.15,
                                                      synthetic.seed(3, i, 0), dev)
            sc, L = w4.w4_lut16_fit(W, 1)
            P, _ = w4.w4_quantize_pack(W, w4.W4_LUT16, scales=sc, codebook=L)
            x = synthetic.normal_bf16_device((1, k), 1.0, synthetic.seed(3, i, 1), dev)
            y = torch.empty((1, n), device=dev)
            ms, how = timed_single([lambda st: w4.w4_gemv(P, x, w4.W4_LUT16, scales=sc,
                                                          codebook=L, y=y, stream=st)],
                                   stream, args.steps, args.warmup)
            b = n * k // 2 + n * (k // 64) * 34 + 2 * k + 4 * n
            print(json.dumps({"target": f"lut16_gemv_m1_{n}x{k}", "ms": ms, "timing": how,
                              "GB/s": b / (ms * 1e-3) / 1e9}), flush=True)
            del W, P, sc, L
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
    log("HBM read ceiling (4 GiB streaming read)")
    ceiling, ms_small = read_ceiling(torch, dev, stream)
    context = {"read_ceiling_4gib_GB/s": round(ceiling, 1),
               "value_frac_of_read_ceiling": round(gbs / ceiling, 4),
               "read_2.25mib_single_call_us": round(ms_small * 1e3, 2)}
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

        # (small calls: timed as the single GEMV calls are)
        quant = [lambda st, m=m: w4.w4_quantize_pack(m["w"], w4.W4_DYADIC, packed=m["packed"],
                                                     scales=m["scales"], stream=st)
                 for m in mats]
        ms_q = timed_single(quant, stream, 3 * len(quant), len(quant))[0] * len(quant)
        rows["quantize_pack_stack"] = {"ms": ms_q, "GB/s": q_bytes / (ms_q * 1e-3) / 1e9}

        outs = [torch.empty((n, k), dtype=torch.bfloat16, device=dev) for n, k in shapes[:7]]
        d_bytes = sum(n * k // 2 + 2 * n * (k // 64) + 2 * n * k for n, k in shapes[:7])

        deq = [lambda st, m=m, o=o: w4.w4_unpack_dequant(m["packed"], w4.W4_DYADIC,
                                                         scales=m["scales"], out=o, stream=st)
               for m, o in zip(mats[:7], outs)]
        ms_d = timed_single(deq, stream, 10 * 35, 70)[0] * len(deq)
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
        # context: the vendor library's dense bf16 GEMM (torch linear) on the
        # same shape with an unquantized bf16 weight
        ms_d = timed(lambda: torch.nn.functional.linear(X, W), stream, 100, 10)
        context["dense_bf16_linear_m256_k8192_n8192_TFLOP/s"] = round(
            2 * 256 * 8192 * 8192 / (ms_d * 1e-3) / 1e12, 1)
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
        ms_v5, how = timed_single([lambda st: w4.w4_gemv(P, xv, w4.W4_DYADIC, scales=S, y=yv,
                                                         stream=st)], stream, args.steps,
                                  args.warmup)
        vb = 8192 * 4096 + 2 * 8192 * 128 + 2 * 8192 + 4 * 8192
        rows["gemv_m1_8192x8192"] = {"ms": ms_v5, "GB/s": vb / (ms_v5 * 1e-3) / 1e9,
                                     "timing": how}
        # the same call over copies of the weight totalling more than the
        # Infinity Cache holds, so each call reads its weight from HBM
        pool = [(P.clone(), S.clone()) for _ in range(rotation_copies(8192 * 4096 + 2 * 8192 * 128))]
        calls = [lambda st, p=p, s=s: w4.w4_gemv(p, xv, w4.W4_DYADIC, scales=s, y=yv, stream=st)
                 for p, s in pool]
        ms_r5, how = timed_single(calls, stream, max(args.steps, 4 * len(pool)), args.warmup)
        rows["gemv_m1_8192x8192_rotating"] = {"ms": ms_r5, "GB/s": vb / (ms_r5 * 1e-3) / 1e9,
                                              "copies": len(pool), "timing": how}
        del pool, calls
        D = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
        ms_d5 = timed(lambda: w4.w4_unpack_dequant(P, w4.W4_DYADIC, scales=S, out=D,
                                                   stream=stream), stream, 50, 5)
        db = 8192 * 4096 + 2 * 8192 * 128 + 2 * 8192 * 8192
        rows["unpack_dequant_8192x8192"] = {"ms": ms_d5, "GB/s": db / (ms_d5 * 1e-3) / 1e9}
        del W, X, P, S, Y, D

    if args.only is None:
        rows.update(other_configs(w4, synthetic, torch, dev, stream, args))
        # context: what a plain device copy reaches on this GPU (read + write)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms_c = timed(lambda: dst.copy_(src), stream, 20, 5)
        context["device_copy_1gib_GB/s_read_plus_write"] = round(
            2 * (1 << 30) / (ms_c * 1e-3) / 1e9, 1)
        del src, dst

    # ---------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(mats, shapes, gbs, rows)

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
        "context": context,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


def cpu_model():
    with open("/proc/cpuinfo") as f:
        for line in f:
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    return "unknown"


def cpu_baseline(mats, shapes, gpu_gbs, rows):
    """The C oracle (oracle/liboracle.c: OpenMP over rows, fp64 sums) timed on
    the host's cores in the same run.  The headline entry is its fused
    dequant + fp64 GEMV over the whole decode stack, on weights the oracle
    quantizes itself (each regenerated on the device and copied to the host;
    quantizing is untimed).  "rows" adds the other workloads: the 2048^2
    GEMV on one thread, quantize_pack and sampled GEMM rows of the 8192^2
    prefill weight, and the k-means fits; each with the GPU:CPU ratio of the
    matching GPU row.  A reported baseline, not a target."""
    import numpy as np
    import torch
    import synthetic
    from oracle import native

    threads = native.num_threads()
    log(f"cpu baseline: C oracle, {threads} threads")

    def host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    def ratio(gpu, cpu):
        return round(gpu / cpu, 1) if gpu and cpu else None

    # headline: fused dequant + fp64 GEMV over all 168 matrices
    nbytes, weights, dt = 0, 0, 0.0
    for i, (n, k) in enumerate(shapes):
        w = synthetic.student_t_bf16_device((n, k), 4, 0.02, synthetic.seed(2, i, 0), "cuda")
        wb = host(w)
        del w
        idx, s = native.dyadic_quantize(wb)
        del wb
        p = np.ascontiguousarray((idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8))
        del idx
        xb = host(mats[i]["x"])
        t0 = time.perf_counter()
        native.dyadic_matmul(p, s, xb)
        dt += time.perf_counter() - t0
        nbytes += n * k // 2 + 2 * n * (k // 64) + 2 * k + 4 * n
        weights += n * k
    value = nbytes / dt / 1e9
    extra = {}

    # the 2048^2 weight (seed 0): quantize + GEMV on one thread
    w = synthetic.normal_bf16_device((2048, 2048), 0.02, synthetic.seed(0, 0, 0), "cuda")
    x = synthetic.normal_bf16_device((1, 2048), 1.0, synthetic.seed(0, 0, 1), "cuda")
    wb, xb = host(w), host(x)
    native.set_num_threads(1)
    t0 = time.perf_counter()
    idx, s = native.dyadic_quantize(wb)
    p = np.ascontiguousarray((idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8))
    tq = time.perf_counter() - t0
    t0 = time.perf_counter()
    native.dyadic_matmul(p, s, xb)
    tg = time.perf_counter() - t0
    native.set_num_threads(threads)
    b = 2048 * 1024 + 2 * 2048 * 32 + 2 * 2048 + 4 * 2048
    g = rows.get("gemv_m1_2048x2048_single_call", {}).get("GB/s")
    extra["gemv_m1_2048x2048_1thread"] = {"GB/s": round(b / tg / 1e9, 4), "cores": 1,
                                          "gpu_ratio": ratio(g, b / tg / 1e9)}
    extra["quantize_2048x2048_1thread"] = {"s": round(tq, 3), "cores": 1}

    # the 8192^2 prefill weight: quantize (all threads), GEMM on 512 sampled rows
    w = synthetic.normal_bf16_device((8192, 8192), 0.02, synthetic.seed(5, 0, 0), "cuda")
    X = synthetic.normal_bf16_device((256, 8192), 1.0, synthetic.seed(5, 0, 1), "cuda")
    wb, Xb = host(w), host(X)
    del w, X
    t0 = time.perf_counter()
    idx, s = native.dyadic_quantize(wb)
    tq = time.perf_counter() - t0
    qb = 2 * 8192 * 8192 + 8192 * 4096 + 2 * 8192 * 128
    g = rows.get("quantize_pack_8192x8192", {}).get("GB/s")
    extra["quantize_pack_8192x8192"] = {"GB/s": round(qb / tq / 1e9, 3), "cores": threads,
                                        "gpu_ratio": ratio(g, qb / tq / 1e9)}
    sel = np.random.default_rng(0).choice(8192, 512, replace=False)
    p = np.ascontiguousarray((idx[sel, 0::2] | (idx[sel, 1::2] << 4)).astype(np.uint8))
    s_sel = np.ascontiguousarray(s[sel])
    del idx
    t0 = time.perf_counter()
    native.dyadic_matmul(p, s_sel, Xb)
    tgm = time.perf_counter() - t0
    tf = 2 * 256 * 512 * 8192 / tgm / 1e12
    g = rows.get("gemm_m256_k8192_n8192", {}).get("TFLOP/s")
    extra["gemm_m256_k8192_512_of_8192_rows"] = {"TFLOP/s": round(tf, 5), "cores": threads,
                                                 "gpu_ratio": ratio(g, tf)}
    del wb, Xb, p

    # k-means fits: one 4096^2 LUT16 weight (3.9B shapes), one 2048^2 SIGNMAG8 weight
    w = synthetic.normal_outliers_bf16_device((4096, 4096), 0.015, 0.001, 0.15,
                                              synthetic.seed(3, 0, 0), "cuda")
    wb = host(w)
    del w
    t0 = time.perf_counter()
    native.lut16_fit(wb, 25)
    tf = time.perf_counter() - t0
    g = rows.get("lut16_fit_4096x4096", {}).get("Mgroups/s")
    mg = 4096 * 64 / tf / 1e6
    extra["lut16_fit_4096x4096"] = {"Mgroups/s": round(mg, 3), "cores": threads,
                                    "gpu_ratio": ratio(g, mg)}
    w = synthetic.student_t_bf16_device((2048, 2048), 5, 0.02, synthetic.seed(4, 0, 0), "cuda")
    wb = host(w)
    del w
    t0 = time.perf_counter()
    native.signmag8_fit(wb, 25)
    tf = time.perf_counter() - t0
    g = rows.get("signmag8_fit_2048x2048", {}).get("Mgroups/s")
    mg = 2048 * 64 / tf / 1e6
    extra["signmag8_fit_2048x2048"] = {"Mgroups/s": round(mg, 3), "cores": threads,
                                       "gpu_ratio": ratio(g, mg)}

    return {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole decode stack ({len(shapes)} matrices, {weights:,} weights): "
                      f"C oracle dequant + fp64 GEMV, OpenMP over rows",
            "cpu_model": cpu_model(), "seconds": round(dt, 2),
            "gpu_ratio": ratio(gpu_gbs, value), "rows": extra}


if __name__ == "__main__":
    main()
