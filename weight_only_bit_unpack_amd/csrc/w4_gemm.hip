// Fused dequant + GEMM for prefill-sized batches (gfx950).
//
// k-means page, section 4.1: batches above the LUT-kernel range go to a mixed
// 4-bit x bf16 kernel.  Y[M][N] = X[M][K] * W_hat[N][K]^T, bf16 MFMA with fp32
// accumulation; the 4-bit weight tile is rebuilt (w4_device.h) straight into
// LDS once per block and k-step, next to the staged activation tile.
//
// Block tile 128 (batch rows) x 64 (weight rows), k-step 64 (one 64-group per
// weight row).  4 waves in a 2 x 2 grid, each 64 x 32 = 4 x 2 tiles of
// v_mfma_f32_16x16x32_bf16.  Both LDS tiles hold each 8-k block in the
// rebuild's slot order, so an MFMA operand is one 16-byte LDS read.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

constexpr int BM = 128, BN = 64, BK = 64;
constexpr int STR = BK / 8 + 1;  // 16-byte units per LDS row (+1 pad against bank conflicts)

template <int CODEC>
__global__ __launch_bounds__(256) void gemm_kernel(GemvProblem P, int M, int y_bf16) {
  constexpr int NPLANES = CODEC == 2 ? 2 : 1;
  __shared__ u32x4 xs[BM * STR];
  __shared__ u32x4 ws[NPLANES][BN * STR];

  const int64_t N = P.n, K = P.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;

  // weight-rebuild role of this thread: row wr, packed dwords 2*wq, 2*wq + 1
  const int wr = tid >> 2, wq = tid & 3;
  const int64_t wrow = n0 + wr;
  const bool wrow_ok = wrow < N;

  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    // activation tile: 128 rows x 8 units
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + 256 * i;
      const int r = u >> 3, uu = u & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < M) v = *reinterpret_cast<const u32x4*>(P.x + (m0 + r) * K + k0 + 8 * uu);
      xs[r * STR + uu] = x_to_sigma(v);
    }
    // weight tile: 64 rows x 8 units, rebuilt from 32 packed bytes per row
    {
      uint32_t p0 = 0x88888888u, p1 = 0x88888888u;
      if (wrow_ok) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(P.packed + wrow * (K >> 1) + (k0 >> 1));
        p0 = src[2 * wq];
        p1 = src[2 * wq + 1];
      }
      u32x4 o0, o1;
      if constexpr (CODEC == 0) {
        const uint32_t sb = wrow_ok ? P.scales[wrow * (K >> 6) + (k0 >> 6)] : 0u;
        const DyadicScale d = dyadic_scale(sb);
        const uint32_t m0c = 0x000F000Fu, m1c = 0x00F000F0u, mg = kMagic;
        if (__builtin_expect(__any(dyadic_scale_is_wide(sb)), 0)) {
          o0 = dyadic_rebuild_wide(p0, d, m0c, m1c, mg);
          o1 = dyadic_rebuild_wide(p1, d, m0c, m1c, mg);
        } else {
          o0 = dyadic_rebuild(p0, d, m0c, m1c, mg);
          o1 = dyadic_rebuild(p1, d, m0c, m1c, mg);
        }
        ws[0][wr * STR + 2 * wq] = o0;
        ws[0][wr * STR + 2 * wq + 1] = o1;
      } else if constexpr (CODEC == 1) {
        u32x4 l0 = {0u, 0u, 0u, 0u}, l1 = l0;
        uint32_t sb = 0;
        if (wrow_ok) {
          const int64_t g = wrow * (K >> 6) + (k0 >> 6);
          const u32x4* lut = reinterpret_cast<const u32x4*>(P.codebook);
          sb = P.scales[g];
          l0 = lut[2 * g];
          l1 = lut[2 * g + 1];
        }
        const Lut16Table t = lut16_table(sb, l0, l1);
        ws[0][wr * STR + 2 * wq] = lut16_rebuild(p0, t);
        ws[0][wr * STR + 2 * wq + 1] = lut16_rebuild(p1, t);
      } else {
        u32x4 c = {0u, 0u, 0u, 0u};
        if (wrow_ok) {
          // dwords 2wq, 2wq+1 cover k 16wq .. 16wq+15: group (k0 + 16 wq) / 32
          const int64_t g = wrow * (K >> 5) + ((k0 + 16 * wq) >> 5);
          c = reinterpret_cast<const u32x4*>(P.codebook)[g];
        }
        const SignMagTable t = signmag_table(c);
        u32x4 h0, l0, h1, l1;
        signmag_rebuild(p0, t, h0, l0);
        signmag_rebuild(p1, t, h1, l1);
        ws[0][wr * STR + 2 * wq] = h0;
        ws[0][wr * STR + 2 * wq + 1] = h1;
        ws[NPLANES - 1][wr * STR + 2 * wq] = l0;
        ws[NPLANES - 1][wr * STR + 2 * wq + 1] = l1;
      }
    }
    __syncthreads();

#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      u32x4 a[4], b[NPLANES][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[(wm * 64 + i * 16 + (lane & 15)) * STR + kb * 4 + (lane >> 4)];
#pragma unroll
      for (int pl = 0; pl < NPLANES; ++pl)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[pl][j] = ws[pl][(wn * 32 + j * 16 + (lane & 15)) * STR + kb * 4 + (lane >> 4)];
#pragma unroll
      for (int pl = 0; pl < NPLANES; ++pl)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x32(a[i], b[pl][j], acc[i][j]);
    }
  }

  // D[m][n] of tile (i, j) sits in lane n + 16 (m / 4), register m % 4
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
        if (r < M) {
          if (y_bf16)
            reinterpret_cast<uint16_t*>(P.y)[r * N + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
          else
            reinterpret_cast<float*>(P.y)[r * N + col] = acc[i][j][e];
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  const dim3 grid((uint32_t)((p.n + BN - 1) / BN), (uint32_t)((m + BM - 1) / BM));
  if (codec == 0)
    gemm_kernel<0><<<grid, dim3(256), 0, stream>>>(p, m, y_bf16);
  else if (codec == 1)
    gemm_kernel<1><<<grid, dim3(256), 0, stream>>>(p, m, y_bf16);
  else
    gemm_kernel<2><<<grid, dim3(256), 0, stream>>>(p, m, y_bf16);
  return hipGetLastError();
}

}  // namespace w4
