// Fused dequant + GEMV for m <= 16 (gfx950).
//
// k-means page, section 4.1: a batch of m <= 16 goes to a dedicated 4-bit
// kernel; section 2.2: the weights are decoded on the fly from a small table.
// DyadicGumbel page, section 2.2: w = step * (idx - 8) per group of 64.
// int4-g32 page, section 5.2: a fused int4 kernel with the group codebook in
// registers.
//
// Work unit: a 16-row x 256-k step.  Lane l = (r = l % 16, q = l / 16) loads
// the 32 packed bytes of row r covering k = 256 s + 64 q .. + 63 (one group
// for the 64-groups, two for SIGNMAG8), so the four q-lanes of a row read one
// full 128-byte line.  Each of the lane's 8 packed dwords is rebuilt into one
// bf16 MFMA B operand (8 values), and v_mfma_f32_16x16x32_bf16 multiplies it
// by the activation operand: A row = batch row m (rows >= m repeat row m-1 and
// are never stored), D[m][r] lands in lane r + 16 (m / 4), register m % 4.
// For m = 1 the matrix core does 16x the necessary multiplies, which is free:
// the kernel is bound by HBM and by the VALU work of the rebuild (about 17
// VALU instructions per 8 weights), and the MFMA takes the multiply-adds off
// the VALU.
//
// The activations are staged once per block into LDS in the rebuild's slot
// order (w4_device.h, SIGMA), in k-chunks when m * k does not fit.
// A block is 4 waves = KSPLIT waves along k x (4 / KSPLIT) row tiles of 16.
// With KSPLIT > 1 the waves' partial sums are added in LDS in a fixed order.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

constexpr int kXsUnits = 2048;  // 32 KiB of LDS for staged activations (16-byte units)

template <int CODEC>
struct Rebuild;

template <>
struct Rebuild<0> {  // DYADIC
  uint32_t sb;
  DyadicScale d;
  __device__ __forceinline__ void load(const GemvProblem& P, int64_t row, int64_t kg, bool valid) {
    sb = valid ? P.scales[row * (P.k >> 6) + (kg >> 6)] : 0u;
    d = dyadic_scale(sb);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const uint32_t (&pw)[8], F&& mma) const {
    const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, mg = kMagic;
    if (__builtin_expect(__any(dyadic_scale_is_wide(sb)), 0)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mma(j, dyadic_rebuild_wide(pw[j], d, m0, m1, mg));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) mma(j, dyadic_rebuild(pw[j], d, m0, m1, mg));
    }
  }
};

template <>
struct Rebuild<1> {  // LUT16
  Lut16Table t;
  __device__ __forceinline__ void load(const GemvProblem& P, int64_t row, int64_t kg, bool valid) {
    u32x4 l0 = {0u, 0u, 0u, 0u}, l1 = l0;
    uint32_t sb = 0;
    if (valid) {
      const int64_t g = row * (P.k >> 6) + (kg >> 6);
      const u32x4* lut = reinterpret_cast<const u32x4*>(P.codebook);
      sb = P.scales[g];
      l0 = lut[2 * g];
      l1 = lut[2 * g + 1];
    }
    t = lut16_table(sb, l0, l1);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const uint32_t (&pw)[8], F&& mma) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(j, lut16_rebuild(pw[j], t));
  }
};

template <>
struct Rebuild<2> {  // SIGNMAG8: two 32-groups per lane step
  SignMagTable t0, t1;
  __device__ __forceinline__ void load(const GemvProblem& P, int64_t row, int64_t kg, bool valid) {
    u32x4 c0 = {0u, 0u, 0u, 0u}, c1 = c0;
    if (valid) {
      const int64_t g = row * (P.k >> 5) + (kg >> 5);
      const u32x4* cb = reinterpret_cast<const u32x4*>(P.codebook);
      c0 = cb[g];
      c1 = cb[g + 1];
    }
    t0 = signmag_table(c0);
    t1 = signmag_table(c1);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const uint32_t (&pw)[8], F&& mma) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 h, l;
      signmag_rebuild(pw[j], j < 4 ? t0 : t1, h, l);
      mma(j, h);
      mma(j, l);
    }
  }
};

__device__ __forceinline__ void locate(const GemvProblem* probs, int count, int64_t b, int& idx) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (probs[mid].tile_begin <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  idx = lo;
}

template <int CODEC, int KSPLIT, bool BATCHED>
__global__ __launch_bounds__(256) void gemv_kernel(GemvProblem single, const GemvProblem* probs,
                                                   int count, int m, int y_bf16) {
  constexpr int RW = 4 / KSPLIT;  // row tiles per block
  __shared__ u32x4 xs[kXsUnits];

  GemvProblem P;
  int64_t blk = blockIdx.x;
  if constexpr (BATCHED) {
    int pi;
    locate(probs, count, blk, pi);
    P = probs[pi];
    blk -= P.tile_begin;
  } else {
    P = single;
  }
  const int64_t N = P.n, K = P.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kw = wave % KSPLIT, rw = wave / KSPLIT;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t row = (blk * RW + rw) * 16 + r16;
  const bool row_ok = row < N;
  const int mr = r16 < m ? r16 : m - 1;  // A row: batch row (padding rows repeat the last)

  // chunk of k staged in LDS: rows of KC/8 units plus one pad unit
  int64_t kc = (int64_t)((kXsUnits / m - 1) / 32) * 256;
  const int64_t kpad = (K + 255) & ~(int64_t)255;
  if (kc > kpad) kc = kpad;
  const int row_units = (int)(kc / 8) + 1;

  const uint8_t* prow = P.packed + row * (K >> 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += kc) {
    const int64_t klen = (K - k0 < kc) ? K - k0 : kc;
    const int steps = (int)((klen + 255) >> 8);
    __syncthreads();
    // stage x[:, k0 : k0 + steps*256] (zero beyond K) in SIGMA order
    const int units = steps * 32;
    for (int u = tid; u < m * units; u += 256) {
      const int mrow = u / units, uu = u - mrow * units;
      const int64_t kk = k0 + 8 * (int64_t)uu;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kk < K) v = *reinterpret_cast<const u32x4*>(P.x + mrow * K + kk);
      xs[mrow * row_units + uu] = x_to_sigma(v);
    }
    __syncthreads();

    for (int s = kw; s < steps; s += KSPLIT) {
      const int64_t kg = k0 + 256 * (int64_t)s + 64 * q;
      const bool ok = row_ok && kg < K;
      u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = a0;
      if (ok) {
        const u32x4* src = reinterpret_cast<const u32x4*>(prow + (kg >> 1));
        a0 = __builtin_nontemporal_load(src);
        a1 = __builtin_nontemporal_load(src + 1);
      }
      Rebuild<CODEC> rb;
      rb.load(P, row, kg, ok);
      const uint32_t pw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const u32x4* xa = &xs[mr * row_units + 32 * s + 8 * q];
      rb.apply(pw, [&](int j, const u32x4& b) { acc = mfma16x16x32(xa[j], b, acc); });
    }
  }

  if constexpr (KSPLIT > 1) {
    __syncthreads();
    float* red = reinterpret_cast<float*>(xs);
    float* mine = red + ((rw * KSPLIT + kw) * 4) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[i * 64 + lane] = acc[i];
    __syncthreads();
    if (kw != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int w = 0; w < KSPLIT; ++w) v += red[((rw * KSPLIT + w) * 4 + i) * 64 + lane];
      acc[i] = v;
    }
  }

  if (!row_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mrow = 4 * q + i;
    if (mrow < m) {
      if (y_bf16)
        reinterpret_cast<uint16_t*>(P.y)[mrow * N + row] = (uint16_t)f32_to_bf16_bits(acc[i]);
      else
        reinterpret_cast<float*>(P.y)[mrow * N + row] = acc[i];
    }
  }
}

template <int CODEC, int KSPLIT>
hipError_t launch_one(const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  const int rows = 16 * (4 / KSPLIT);
  const int64_t blocks = (p.n + rows - 1) / rows;
  gemv_kernel<CODEC, KSPLIT, false><<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      p, nullptr, 0, m, y_bf16);
  return hipGetLastError();
}

template <int CODEC>
hipError_t launch_codec(const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  switch (gemv_pick_ksplit(p.n, p.k, m)) {
    case 1: return launch_one<CODEC, 1>(p, m, y_bf16, stream);
    case 2: return launch_one<CODEC, 2>(p, m, y_bf16, stream);
    default: return launch_one<CODEC, 4>(p, m, y_bf16, stream);
  }
}

}  // namespace

int gemv_rows_per_block(int ksplit) { return 16 * (4 / ksplit); }

int gemv_pick_ksplit(int64_t n, int64_t k, int m) {
  (void)k;
  (void)m;
  // enough blocks of 64 rows to give every CU several: no k split
  if ((n + 63) / 64 >= 1024) return 1;
  if ((n + 31) / 32 >= 1024) return 2;
  return 4;
}

hipError_t launch_gemv(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  if (codec == 0) return launch_codec<0>(p, m, y_bf16, stream);
  if (codec == 1) return launch_codec<1>(p, m, y_bf16, stream);
  return launch_codec<2>(p, m, y_bf16, stream);
}

hipError_t launch_gemv_batched(int codec, const GemvProblem* probs_dev, int count,
                               int64_t total_blocks, int m, int y_bf16, hipStream_t stream) {
  GemvProblem none{};
  const dim3 grid((uint32_t)total_blocks), block(256);
  if (codec == 0)
    gemv_kernel<0, 1, true><<<grid, block, 0, stream>>>(none, probs_dev, count, m, y_bf16);
  else if (codec == 1)
    gemv_kernel<1, 1, true><<<grid, block, 0, stream>>>(none, probs_dev, count, m, y_bf16);
  else
    gemv_kernel<2, 1, true><<<grid, block, 0, stream>>>(none, probs_dev, count, m, y_bf16);
  return hipGetLastError();
}

}  // namespace w4
