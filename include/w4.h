/*
 * w4.h -- C ABI of the MI355X (gfx950) group-wise 4-bit weight library.
 *
 * The operation comes from three pages on weight-only 4-bit quantization:
 *
 *  [DG]  "MiniCPM5-1B 验证: 6× 压缩 ... 50ms Triton 推理" (DyadicGumbel 4-bit):
 *        sec. 2.1 dyadic codebook step*{-8..7} with step = scale/8;
 *        sec. 2.2 blocks of 64 weights, one bf16 scale each, reconstruction
 *        w = step*(idx - 8); sec. 2.3/2.5 hard argmin to a 4-bit index, two
 *        indices per byte as (lo | hi << 4), unpack + rebuild to bf16 per layer.
 *  [KM]  "K-Means量化技术：突破LLM低比特部署瓶颈": sec. 1.2 per-block (64)
 *        16-centre 1D k-means codebook + 16-bit scale, nearest-centre index;
 *        sec. 2.2 decode by table lookup; sec. 4.1 kernel choice by batch m
 *        (a LUT kernel for m <= 16, a mixed 4-bit kernel up to 256).
 *  [G32] "int4-g32+warm 裸量化：原理与实验报告": sec. 1.2 the transform
 *        families of the warm start; sec. 1.3 nearest of 8 levels per group
 *        of 32 with a separate sign bit, Lloyd refinement; sec. 2 1 sign bit +
 *        3-bit level index per weight, dense fp16 rebuild or a fused int4
 *        kernel with the 8-value codebook in registers.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers owned by the caller, all on the current
 *    device (hipSetDevice), as is `stream`; the library keeps none of them
 *    after returning.  It allocates no memory, except w4_gemm and
 *    w4_gemv with m >= 2, which keep a device workspace per (device, stream)
 *    for the process's life (see there).
 *  - `stream` is a hipStream_t (NULL = the null stream).  A call only enqueues
 *    work on it; it never synchronises the stream or the device.
 *  - All validation happens on the host before anything is enqueued.  On any
 *    error return nothing is enqueued and no output byte changes.  Faults in
 *    the kernels surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give the same output bits
 *    (fixed reduction order, no atomics).
 *  - Weights are row-major [n][k] (n = output features, k = input features,
 *    the layout of a PyTorch Linear weight).  A group is `group` consecutive
 *    weights along k; k must be a multiple of the codec's group (64, or 32
 *    for SIGNMAG8) in the quantize, dequant and fit calls, and a multiple of
 *    64 for every codec in the matrix calls (w4_gemv, w4_gemm, w4_linear and
 *    the batched GEMV), whose kernels step over k in 64-weight units.
 *  - Preconditions that are not checked: finite inputs; buffers contiguous,
 *    of the sizes stated, and not overlapping one another.
 *
 * Quantized weight = three planar row-major arrays
 *   packed   uint8 [n][k/2]  nibble(r, c) = (packed[r][c/2] >> (4*(c%2))) & 15
 *   scales   bf16  [n][k/64] DYADIC, LUT16, LUT16S;   NULL for SIGNMAG8
 *   codebook LUT16:    bf16 [n][k/64][16] normalised levels L_j;
 *            LUT16S:   bf16 [16] normalised levels L_j shared by every group;
 *            DYADIC5:  uint8 [n][k/8] high-bit plane (passed as codebook):
 *                      per run of 32 weights k = 32c .. 32c+31 a little-endian
 *                      32-bit word M; the 5-bit index of weight 32c + i is
 *                      nibble | (M >> bit(i) & 1) << 4 with, for d = i / 8 and
 *                      e = i % 8, bit(i) = P[e] + A[2d + (e % 4 >= 2)],
 *                      P = {4, 8, 4, 8, 20, 24, 20, 24},
 *                      A = {-4, -3, -2, -1, 4, 5, 6, 7};
 *                      the nibble plane holds the low 4 bits;
 *            SIGNMAG8: fp16 [n][k/32][8]  magnitudes M_j;    NULL for DYADIC
 * Reconstruction (w_hat, "dequantized weight"):
 *   DYADIC:   w_hat = RNE_bf16((s/8) * (nib - 8))    a zero result is +0.0
 *   LUT16, LUT16S: w_hat = RNE_bf16(s * L[nib])
 *   DYADIC5:  w_hat = RNE_bf16((s/16) * (j5 - 16))  an exact zero is +0.0
 *   SIGNMAG8: w_hat = (nib & 8 ? -1 : +1) * M[nib & 7]    (fp16, exact)
 * (RNE = round to nearest, ties to even.)
 */
#ifndef W4_H
#define W4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_EINVAL = 1,       /* NULL pointer for a non-empty buffer, bad enum, negative size */
  W4_ESHAPE = 2,       /* k not a multiple of the call's group, m outside the call's
                          range, or a size above the call's stated limit               */
  W4_EALIGN = 3,       /* a pointer not aligned as the call states                      */
  W4_EUNSUPPORTED = 4, /* a codec / dtype combination the call does not provide         */
  W4_EHIP = 5          /* the kernel launch failed (hipGetLastError)                    */
} w4_status;

/* W4_LUT16S: the LUT16 rebuild with one 16-level table for the whole weight
 * and a bf16 scale per group of 64 -- 4.25 bits per weight plus 32 bytes, the
 * size [KM] sec. 2.1 states for its 3.9B model (about 2.1 GB).  The table is
 * an input; the oracle fits it by k-means over the whole weight. */
/* W4_DYADIC5: [DG] sec. 2.1's dyadic codes at b = 3, 4 and 5 bits in one
 * 5-bit index space (the b-bit code j is the 5-bit code j * 2^(5-b)), so a
 * group's width only restricts which codes it may take; see
 * w4_quantize_dyadic5.  Reconstruction RNE_bf16((s/16) * (j5 - 16)). */
/* [KM] sec. 2.2 decodes by looking up precomputed values of every byte and
 * stores the scales with the indices.  The W4_LUT16S batched GEMV on 64-row
 * tiles decodes a packed byte at a time through a 256-entry table of level
 * pairs (L[b & 15], L[b >> 4]) that each block builds in LDS; its single
 * calls and its batches of short tiles decode per nibble as W4_LUT16S_PERM,
 * measured as fast or faster there.  The two decodes give the matrix core the
 * same products in a different order within each group of 8 weights, so
 * their results agree within the GEMV tolerance but not always bit for bit.
 * Two variants are kept for comparison:
 * W4_LUT16S_PERM: the LUT16S storage and results, with a GEMV that always
 *   looks the levels up per nibble from byte-plane tables with v_perm, as
 *   LUT16 does.  Every other call treats it exactly as W4_LUT16S.
 * W4_LUT16S_IL: the LUT16S weight with each row's scales interleaved into its
 *   packed bytes (k a multiple of 256): per 256-k block a 144-byte record of
 *   the block's 128 packed bytes, its four bf16 scales and 8 zero bytes, so
 *   `packed` is uint8 [n][k/256 * 144] and `scales` is unused.  Built from the
 *   planar arrays by w4_lut16s_interleave; taken by w4_gemv and the batched
 *   GEMV (decoded through the pair table, within the GEMV tolerance of
 *   W4_LUT16S as above); the other calls return
 *   W4_EUNSUPPORTED. */
typedef enum {
  W4_DYADIC = 0,
  W4_LUT16 = 1,
  W4_SIGNMAG8 = 2,
  W4_LUT16S = 3,
  W4_DYADIC5 = 4,
  W4_LUT16S_PERM = 5,
  W4_LUT16S_IL = 6
} w4_codec;

/* Largest k of a matrix product call: keeps every per-block byte offset of the
 * kernels within 32 bits. */
#define W4_MAX_MATMUL_K 4194304
/* Largest Lloyd round count the fit calls accept. */
#define W4_MAX_FIT_ITERS 1024
typedef enum { W4_F32 = 0, W4_BF16 = 1, W4_F16 = 2 } w4_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* w4_status_str(int32_t status);

/* Weights per group of a codec: 64 (DYADIC, LUT16, LUT16S and its variants,
 * DYADIC5), 32 (SIGNMAG8); -1 if unknown. */
int32_t w4_group_size(int32_t codec);

/*
 * w4_quantize_pack -- quantize a bf16 weight [n][k] and pack two 4-bit indices
 * per byte.  [DG] sec. 2.1-2.3, 2.5; [KM] sec. 1.2; [G32] sec. 1.3 step 4.
 *   DYADIC:   writes scales[r][g] = max |w| over the group (a bf16 value), then
 *             idx = the lowest j minimising |w - (s/8)(j-8)| over the exact
 *             codes; an all-zero group gets s = +0 and idx 8.  codebook: NULL.
 *   LUT16:    reads scales (bf16 [n][k/64]) and codebook (bf16 [n][k/64][16]);
 *             idx = the lowest j minimising the exact distance |w - s*L_j|
 *             (the levels s*L_j as exact real products), for every finite
 *             weight, scale and table: also weights beyond the levels' range
 *             and levels far apart in magnitude.
 *   LUT16S:   as LUT16 with the one table codebook (bf16 [16]) for every group.
 *   DYADIC5:  not provided here (W4_EUNSUPPORTED): w4_quantize_dyadic5 writes
 *             both of its index planes.
 *   SIGNMAG8: reads codebook (fp16 [n][k/32][8], finite or +inf, the fit's
 *             output beyond the fp16 range); scales: NULL;
 *             nibble = (w < 0) << 3 | the lowest j minimising the exact
 *             ||w| - M_j| (a +inf magnitude is never nearer than a finite one;
 *             a group of only +inf magnitudes gives index 0).
 * w: bf16 [n][k], 16-byte aligned.  packed: uint8 [n][k/2], 16-byte aligned.
 * scales: 2-byte aligned.  codebook: 16-byte aligned.
 * n == 0 or k == 0: nothing to do, returns W4_OK.
 */
w4_status w4_quantize_pack(int32_t codec, int64_t n, int64_t k, const uint16_t* w,
                           uint8_t* packed, uint16_t* scales, const uint16_t* codebook,
                           void* stream);

/*
 * w4_unpack_dequant -- rebuild the dense weight.  [DG] sec. 2.2, 2.5 (unpack
 * kernel: packed byte -> nibble split -> step -> bf16); [KM] sec. 2.2 (LUT
 * decode); [G32] sec. 2 (dense fp16 weight).
 * out: bf16 [n][k] for DYADIC, LUT16, LUT16S and DYADIC5, fp16 [n][k] for
 * SIGNMAG8; 16-byte aligned.
 * packed and codebook 16-byte aligned, scales 2-byte aligned.
 */
w4_status w4_unpack_dequant(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                            const uint16_t* scales, const uint16_t* codebook, void* out,
                            void* stream);

/*
 * w4_quantize_dyadic5 -- quantize a bf16 weight [n][k] to W4_DYADIC5 with a
 * width b in {3, 4, 5} bits per group of 64.  [DG] sec. 2.1 (codes
 * (s/half)(j - half), half = 2^(b-1); the 3/4/5-bit codebooks share one index
 * space), sec. 2.2 (scale = the group's absmax here, as for W4_DYADIC).
 * For each group: s = max |w| (bf16, exact), written to scales; each weight
 * takes the lowest j minimising |w - (s/half)(j - half)| over the group's
 * 2^b exact codes and is stored as j5 = j * 2^(5-b); an all-zero group gets
 * s = +0 and j5 = 16.  The widths choose the precision per group (the pages
 * give no rule for choosing them); widths == NULL means 5 bits everywhere,
 * and a width other than 3 or 4 means 5.
 * w: bf16 [n][k], 16-byte aligned.  widths: uint8 [n][k/64] or NULL.
 * packed: uint8 [n][k/2] (low 4 bits of j5), 16-byte aligned.  msb: uint8
 * [n][k/8] high-bit plane (layout at the top of this header), 16-byte
 * aligned.  scales: bf16 [n][k/64], 2-byte aligned.
 * Errors: W4_EINVAL (negative size, null pointer), W4_ESHAPE (k % 64 != 0),
 * W4_EALIGN.
 */
w4_status w4_quantize_dyadic5(int64_t n, int64_t k, const uint16_t* w, const uint8_t* widths,
                              uint8_t* packed, uint8_t* msb, uint16_t* scales, void* stream);

/*
 * w4_lut16s_interleave -- the W4_LUT16S_IL layout of a W4_LUT16S weight
 * [n][k]: out[r] holds, for each 256-k block j, packed[r][128 j .. 128 j + 127],
 * then scales[r][4 j .. 4 j + 3] (bf16, little-endian), then 8 zero bytes.
 * [KM] sec. 2.2 (scales interleaved with the indices).
 * packed: uint8 [n][k/2], 16-byte aligned; scales: bf16 [n][k/64], 2-byte
 * aligned; out: uint8 [n][k/256 * 144], 16-byte aligned.
 * Errors: W4_EINVAL (negative size, null pointer), W4_ESHAPE (k % 256 != 0),
 * W4_EALIGN.
 */
w4_status w4_lut16s_interleave(int64_t n, int64_t k, const uint8_t* packed,
                               const uint16_t* scales, uint8_t* out, void* stream);

/*
 * w4_lut16_fit -- fit the LUT16 side tables of a bf16 weight [n][k]: per group
 * of 64, a scale and 16 levels by 1D k-means.  [KM] sec. 1.2 (per-block 16-
 * centre k-means, 16-bit scale); [G32] sec. 1.3 (quantile start, 25 rounds).
 * For each group, in fp64:
 *   s = max |w| (written to scales as bf16; exact), u = w / s;
 *   start: the elements of rank 4q + 2 (q = 0..15) in a stable ascending sort
 *          of u (equal values keep element order);
 *   `iters` rounds: assign each u to the centre with the smallest |u - c|,
 *          the lowest centre on a tie; each centre with members becomes the
 *          sum of its members, added in increasing element order, divided by
 *          their count; a centre without members keeps its value;
 *   codebook[r][g][q] = c_q rounded to bf16 (nearest, ties to even).
 * An all-zero group gets scale +0 and 16 levels +0.  The result is bit-exact:
 * every step is an exact operation or one IEEE fp64 operation in a fixed
 * order.  The outputs are the scales / codebook inputs of w4_quantize_pack
 * and the matrix calls for W4_LUT16.
 * w: bf16 [n][k], 16-byte aligned; finite values.  scales: bf16 [n][k/64],
 * 2-byte aligned.  codebook: bf16 [n][k/64][16], 16-byte aligned.
 * iters: 0 .. W4_MAX_FIT_ITERS (0: the quantile start itself).
 * Errors: W4_EINVAL (negative size, iters out of range, null pointer),
 * W4_ESHAPE (k % 64 != 0, or more than 16 * (2^31 - 1) groups), W4_EALIGN.
 */
w4_status w4_lut16_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* scales,
                       uint16_t* codebook, int32_t iters, void* stream);

/*
 * w4_signmag8_fit -- fit the W4_SIGNMAG8 magnitudes of a bf16 weight [n][k]:
 * per group of 32, 8 levels by 1D k-means on the magnitudes.  [G32] sec. 1.3
 * (groups of 32, |w| clustered into 8 magnitudes by Lloyd rounds from a
 * quantile start, 25 rounds, fp16 codebook).
 * For each group, in fp64: a = |w|;
 *   start: the elements of rank 4q + 2 (q = 0..7) in an ascending sort of a;
 *   `iters` rounds as in w4_lut16_fit (nearest centre, lowest on a tie; the
 *          members' sum in increasing element order over their count; a
 *          centre without members keeps its value);
 *   codebook[r][g][q] = c_q rounded to fp16 (nearest, ties to even; at or
 *          above 65520 the result is +inf).
 * Bit-exact like w4_lut16_fit.  The output is the codebook input of
 * w4_quantize_pack and the matrix calls for W4_SIGNMAG8 (those need k % 64 == 0).
 * w: bf16 [n][k], 16-byte aligned; finite values.  codebook: fp16 [n][k/32][8],
 * 16-byte aligned.  iters: 0 .. W4_MAX_FIT_ITERS.
 * Errors: W4_EINVAL (negative size, iters out of range, null pointer),
 * W4_ESHAPE (k % 32 != 0, or more than 32 * (2^31 - 1) groups), W4_EALIGN.
 */
w4_status w4_signmag8_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                          int32_t iters, void* stream);

/*
 * w4_signmag8_fit_warm -- fit the W4_SIGNMAG8 magnitudes with the warm start:
 * per group of 32, the best of 112 parametric transforms gives 8 starting
 * levels, then Lloyd rounds as in w4_signmag8_fit.  [G32] sec. 1.2 (the two
 * transform families and their inverses), 1.3 steps 1-3, 5.1 (the per-group
 * procedure), 2 (the 8-bit per-group parameter code).
 * For each group, in fp64, with a = |w| and gmax = max a:
 *   candidates in increasing code (the lowest code wins a tie):
 *     rational, code = b_idx << 3 | beta_idx: f(a) = a / (b + a^beta) with
 *       b = 10^((5 b_idx - 42) / 14) * gmax (b_idx 0..14) and beta =
 *       {0.50, 0.55, 0.65, 0.75, 0.85, 0.95, 1.00}[beta_idx];
 *     tanh, code = 128 | b_idx << 3: f(a) = tanh(a / b), b =
 *       {0.25, 0.4, 0.6, 0.85, 1.2, 1.8, 3.0}[b_idx] * gmax;
 *   per candidate: fmax = f(gmax); q_i = rint((f(a_i) / fmax) * 7) in 0..7;
 *     levels L_q = f^-1((q / 7) * fmax) (rational beta = 1: fd*b / (1 - fd);
 *     beta < 1: the root of w = fd*b + fd*w^beta; tanh: b * atanh(fd));
 *     error = sum over i in element order of (a_i - L_{q_i})^2;
 *   the winner's 8 levels start `iters` Lloyd rounds on a; codebook = the
 *   levels rounded to fp16; params (if not NULL) = the winner's code.
 * An all-zero group gets 8 zero levels and code 0.  pow, tanh and atanh are
 * the device math library's, within a few ulps of the exact functions: the
 * result can differ from another implementation of the same steps in the
 * last bits of a level, and so, on a near-tie of two candidates' errors, in
 * the candidate chosen.
 * w: bf16 [n][k], 16-byte aligned; finite values.  codebook: fp16
 * [n][k/32][8], 16-byte aligned.  params: uint8 [n][k/32] or NULL.
 * iters: 0 .. W4_MAX_FIT_ITERS.
 * Errors: W4_EINVAL (negative size, iters out of range, null w or codebook),
 * W4_ESHAPE (k % 32 != 0, or more than 2 * (2^31 - 1) groups), W4_EALIGN.
 */
w4_status w4_signmag8_fit_warm(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                               uint8_t* params, int32_t iters, void* stream);

/*
 * w4_gemv -- fused dequant + matrix-vector product for small batches,
 * y[i][r] = sum_c x[i][c] * w_hat[r][c], accumulated in fp32.  [KM] sec. 4.1
 * (m <= 16 goes to the LUT kernel), sec. 2.2; [G32] sec. 5.2 (fused kernel with
 * the codebook in registers).
 * x: bf16 [m][k], 16-byte aligned.  m: 1..16 (m == 0: nothing to do).
 * y: [m][n] of y_dtype W4_F32 (4-byte aligned) or W4_BF16 (RNE, 2-byte aligned).
 * The result is within 1e-3 * sum_c |x w_hat| + 1e-6 of the exact sum (bf16 y:
 * plus its own rounding, 2^-8 |y|), and the same inputs always give the same
 * bits.  The bound follows from the fp32 sums alone for k <= 16760; above
 * that it rests on the matrix core summing each instruction's products
 * before adding them to the accumulator (tested to k = 65600).
 * k == 0 (with m, n > 0): y = +0.
 * Workspace: with m >= 2 and n <= 65536 the call may split k into S <= 32
 * slices across blocks and enqueue a second kernel that adds the slices' fp32
 * partial sums in slice order; the partials use a device buffer of
 * S * m * n * 4 bytes that the library keeps per (device, stream) exactly as
 * for w4_gemm (see there).  m == 1 uses none.
 * Additional error: W4_EHIP when that buffer cannot be allocated.
 */
w4_status w4_gemv(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                  const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                  int32_t m, void* y, int32_t y_dtype, void* stream);

/*
 * w4_gemm -- fused dequant + matrix product for prefill-sized batches,
 * Y[i][r] = sum_c X[i][c] * w_hat[r][c] with bf16 MFMA and fp32 accumulation;
 * the weight tiles are rebuilt into LDS.  [KM] sec. 4.1 (the 4-bit mixed kernel
 * band, m up to 256).  Same arguments, tolerance and determinism as w4_gemv;
 * m >= 1 (tuned for m >= 128).  k == 0 (with m, n > 0): y = +0.
 * Workspace: the call enqueues up to three kernels (an activation re-layout,
 * the product, and an in-order sum of the k-split partials) that use a device
 * buffer of ceil(m/B) * B * k * 2 bytes plus, when k is split S <= 8 ways,
 * S * ceil(m/B) * B * ceil(n/128) * 128 * 4 bytes, where B, the batch rows
 * of a block, is 128 when m <= 128, k is a multiple of 128 and the codec is
 * not SIGNMAG8, and 256 otherwise.  The library keeps one such buffer per
 * (device, stream): allocated with hipMalloc on first use, replaced by a new
 * one at least twice as large when a call needs more.  Replaced buffers are
 * never freed (work enqueued earlier, or a graph captured earlier, may still
 * use them), so growing never waits for the stream; nothing is freed before
 * the process ends, also for streams the caller destroys.  Calls on one
 * stream are ordered and share the buffer; calls on different streams never
 * do.
 * Graph capture: a call that would create or grow the buffer cannot be
 * captured (hipMalloc); make one call of each shape to be captured on the
 * capture stream before capturing.  After that, calls only enqueue kernels
 * (no memset, no allocation).  A captured graph keeps using the buffer of
 * its capture stream whatever stream it is replayed on: replays must not
 * overlap one another or eager calls on the capture stream.
 * Additional error: W4_EHIP when the workspace cannot be allocated.
 */
w4_status w4_gemm(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                  const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                  int32_t m, void* y, int32_t y_dtype, void* stream);

/*
 * w4_gemm_noalloc -- w4_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture without a warm-up call, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results (bit for bit)
 * and errors as w4_gemm, but the workspace is a fixed device array of
 * W4_NOALLOC_SCRATCH_BYTES that the library defines and every GPU it runs on
 * holds until the process ends; the call itself calls no allocating routine.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or replays of graphs that contain this call) race
 * and must be ordered by the caller.  Nothing in the array needs to start at
 * zero: each call writes the parts it reads.
 * Additional error: W4_ESHAPE when the call's workspace (the w4_gemm sizes)
 * exceeds W4_NOALLOC_SCRATCH_BYTES, e.g. m = 256 with k = n = 8192 needs
 * 36 MiB.
 */
#define W4_NOALLOC_SCRATCH_BYTES (64u << 20)
w4_status w4_gemm_noalloc(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                          const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                          int32_t m, void* y, int32_t y_dtype, void* stream);

/*
 * w4_linear -- the linear layer with the kernel chosen by batch size, as
 * [KM] sec. 4.1 lays out: m <= 16 -> w4_gemv (the table-lookup kernel),
 * larger m -> w4_gemm (the mixed 4-bit x bf16 MFMA kernel; the page's further
 * switch to a plain bf16 GEMM above m = 256 is not taken, as w4_gemm serves
 * every m).  Same arguments, results and errors as the call it selects.
 */
w4_status w4_linear(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                    const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                    int32_t m, void* y, int32_t y_dtype, void* stream);

/*
 * Batched GEMV: one launch over many independent w4_gemv problems of one codec
 * and one m (e.g. every linear layer of a decode step whose inputs are ready).
 * [DG] sec. 2.5 runs one unpack launch per layer, 168 per forward; one launch
 * for all of them removes the per-launch ramp.
 *
 * 1. Fill a HOST array of count w4_gemv_problem records (tile_begin is
 *    ignored) and call w4_gemv_batched_plan: it validates every problem
 *    exactly as w4_gemv would, writes each tile_begin (an opaque work offset;
 *    problems with larger k get earlier work) and fills *info.
 * 2. Copy the count records byte for byte into device memory (16-byte
 *    aligned).  The table is only read, so it can be launched any number of
 *    times; each launch writes every problem's y, so launches that overlap
 *    in time write the same outputs and must be ordered by the caller if
 *    anything reads or changes those buffers in between.
 * 3. Call w4_gemv_batched with that device table and the plan's info.  The
 *    kernel trusts the device copy: it must equal an array the plan accepted.
 * Errors: W4_EINVAL / W4_ESHAPE / W4_EALIGN / W4_EUNSUPPORTED as for w4_gemv
 * (the plan reports the first failing problem's status and writes nothing to
 * *info); W4_ESHAPE when the problems need more than 2^31 - 1 tiles;
 * w4_gemv_batched returns W4_EINVAL when m differs from info->m or
 * info->tile_rows is not one the plan can choose.
 */
typedef struct {
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* codebook;
  const uint16_t* x; /* bf16 [m][k] */
  void* y;           /* [m][n] of the call's y_dtype */
  int64_t n;
  int64_t k;
  int64_t tile_begin; /* written by w4_gemv_batched_plan */
} w4_gemv_problem;

typedef struct {
  int64_t total_tiles; /* work tiles over all problems */
  int64_t k_min;       /* smallest k */
  int64_t k_max;       /* largest k (sizes the kernel's LDS) */
  int32_t count;       /* number of problems */
  int32_t m;           /* the plan's m; w4_gemv_batched must be called with it */
  int32_t tile_rows;   /* rows per work tile: 64, or 32 / 16 (m == 1 only)
                          when 64-row tiles would give fewer than 1024 */
  int32_t flags;       /* bit 0: some problem's k is not a multiple of 256
                          (the kernel then zeroes the lanes past its k;
                          W4_LUT16S_IL, whose k must be, gets W4_ESHAPE);
                          written by the plan like the rest of the record */
} w4_gemv_batch_info;

w4_status w4_gemv_batched_plan(int32_t codec, int32_t m, int32_t y_dtype,
                               w4_gemv_problem* problems_host, int32_t count,
                               w4_gemv_batch_info* info);

w4_status w4_gemv_batched(int32_t codec, int32_t m, int32_t y_dtype,
                          w4_gemv_problem* problems_device, const w4_gemv_batch_info* info,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
