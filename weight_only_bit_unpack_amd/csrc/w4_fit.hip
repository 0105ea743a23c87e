// Per-group 16-level LUT fitting for the LUT16 codec (gfx950).
//
// k-means page, section 1.2: every block of 64 weights gets its own 1D k-means
// clustering with 16 centres and a scale.  int4-g32 page, section 1.3: the
// Lloyd step starts from quantiles of the group and runs 25 rounds.
//
// For one group (w_0 .. w_63, bf16):
//   s   = max |w_i| (a bf16 value, written as the group's scale);
//   u_i = w_i / s in fp64 (s = 0: scale +0 and all levels +0);
//   start: sort u stably (equal values keep element order) and take the
//          elements of sorted rank 4q + 2 as centres c_0 .. c_15;
//   each round: assign every u_i to the centre with the smallest |u_i - c_q|
//          (the lowest q on a tie); move every centre with members to the
//          fp64 sum of its members, added in increasing element order,
//          divided by their count; a centre with no members stays put;
//   levels: L_q = c_q rounded to bf16 (nearest, ties to even).
// Every step is exact or one IEEE fp64 operation in a fixed order, so the
// result is the same bits on any device and in the CPU reference.
//
// Work layout: 16 lanes per group (lane j holds elements 4j .. 4j+3 and owns
// centre j), four groups per wave, 16 groups per 256-thread block; the
// group's u, centres and assignments live in LDS.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

constexpr int kFitGroups = 16;  // groups per block
constexpr int kUPad = 65;       // doubles per group row in LDS (pad: groups in different banks)

// fp64 -> bf16 bits, round to nearest, ties to even; subnormal results on the
// 2^-133 grid, overflow to infinity.  Finite inputs only.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  const int E = (int)(a >> 52);
  if (E == 0) return sign;  // zero or fp64 subnormal: far below half the bf16 quantum
  const int e = E - 1023;                    // value = S * 2^(e - 52)
  const uint64_t S = (a & 0x000FFFFFFFFFFFFFull) | (1ull << 52);
  const int q = e - 7 > -133 ? e - 7 : -133;  // exponent of the result's last bit
  const int shift = q - e + 52;               // >= 45
  if (shift >= 60) return sign;               // value < 2^(q - 7): rounds to zero
  uint64_t R = S >> shift;
  const uint64_t rem = S & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (R & 1))) ++R;
  if (R == 0) return sign;
  // value = R * 2^q with R <= 256 (R >= 128 unless q = -133)
  const int64_t bits = ((int64_t)(q + 133) << 7) + (int64_t)R;
  return (uint16_t)(sign | (bits >= 0x7F80 ? 0x7F80 : (uint16_t)bits));
}

__global__ __launch_bounds__(256) void lut16_fit_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                        int64_t k, int iters,
                                                        uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ lut) {
  __shared__ double su[kFitGroups][kUPad];
  __shared__ double sc[kFitGroups][16];
  __shared__ uint8_t sa[kFitGroups][64];
  const int tid = threadIdx.x, gl = tid >> 4, j = tid & 15;
  const int64_t g = k >> 6, total = n * g;
  const int64_t t = (int64_t)blockIdx.x * kFitGroups + gl;
  const bool valid = t < total;

  double u[4] = {0.0, 0.0, 0.0, 0.0};
  if (valid) {
    const int64_t r = t / g, gi = t - r * g;
    const uint2 v = *reinterpret_cast<const uint2*>(w + r * k + gi * 64 + 4 * j);
    const uint32_t h[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (double)__uint_as_float(h[e] << 16);
  }
  // group absmax over the 16 lanes (exact)
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = fabs(u[e]) > s ? fabs(u[e]) : s;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    const double other = __shfl_xor(s, o, 16);
    s = other > s ? other : s;
  }
  const bool zero = !(s > 0.0);
  if (!zero) {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = u[e] / s;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) su[gl][4 * j + e] = u[e];
  __syncthreads();

  // quantile start: stable rank of each element; ranks 4q + 2 become centres
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int me = 4 * j + e;
    int rank = 0;
    for (int i = 0; i < 64; ++i) {
      const double v = su[gl][i];
      rank += (v < u[e] || (v == u[e] && i < me)) ? 1 : 0;
    }
    if ((rank & 3) == 2) sc[gl][rank >> 2] = u[e];
  }
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    double c[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) c[q] = sc[gl][q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int best = 0;
      double bd = fabs(u[e] - c[0]);
#pragma unroll
      for (int q = 1; q < 16; ++q) {
        const double d = fabs(u[e] - c[q]);
        if (d < bd) {
          bd = d;
          best = q;
        }
      }
      sa[gl][4 * j + e] = (uint8_t)best;
    }
    __syncthreads();
    // centre j: its members in increasing element order
    double sum = 0.0;
    int cnt = 0;
    for (int i = 0; i < 64; ++i) {
      const bool mine = sa[gl][i] == j;
      const double v = su[gl][i];
      sum = mine ? sum + v : sum;
      cnt += mine ? 1 : 0;
    }
    if (cnt > 0) sc[gl][j] = sum / (double)cnt;
    __syncthreads();
  }

  if (valid) {
    lut[t * 16 + j] = zero ? (uint16_t)0 : f64_to_bf16_rne(sc[gl][j]);
    if (j == 0) scales[t] = f64_to_bf16_rne(s);  // s is a bf16 value: exact
  }
}

}  // namespace

hipError_t launch_lut16_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* scales,
                            uint16_t* lut, int iters, hipStream_t stream) {
  const int64_t groups = n * (k / 64);
  const int64_t blocks = (groups + kFitGroups - 1) / kFitGroups;
  lut16_fit_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(w, n, k, iters, scales, lut);
  return hipGetLastError();
}

}  // namespace w4
