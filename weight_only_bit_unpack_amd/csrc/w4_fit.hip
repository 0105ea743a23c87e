// Per-group k-means fitting of the LUT codecs' tables (gfx950).
//
// k-means page, section 1.2: every block of 64 weights gets its own 1D k-means
// clustering with 16 centres and a scale.  int4-g32 page, section 1.3: groups
// of 32 weights, their magnitudes clustered into 8 levels by Lloyd rounds from
// a start; the quantile start and the 25 rounds are used for both.
//
// LUT16 (groups of 64, 16 centres), for one group w_0 .. w_63 (bf16):
//   s   = max |w_i| (a bf16 value, written as the group's scale);
//   u_i = w_i / s in fp64 (s = 0: scale +0 and all levels +0);
//   levels: L_q = c_q rounded to bf16 (nearest, ties to even).
// SIGNMAG8 (groups of 32, 8 centres): u_i = |w_i| in fp64, no scale; the
//   magnitudes M_q = c_q rounded to fp16 (nearest, ties to even).
// Both, from u:
//   start: sort u stably (equal values keep element order) and take the
//          elements of sorted rank 4q + 2 as centres c_q;
//   each round: assign every u_i to the centre with the smallest |u_i - c_q|
//          (the lowest q on a tie); move every centre with members to the
//          fp64 sum of its members, added in increasing element order,
//          divided by their count; a centre with no members stays put.
// Every step is exact or one IEEE fp64 operation in a fixed order, so the
// result is the same bits on any device and in the CPU reference.
//
// Work layout: one lane per centre (16 or 8 lanes per group), each lane
// holding four of the group's elements (lane j: elements 4j .. 4j+3); 256
// threads hold 16 or 32 groups; the group's u, centres and assignments live
// in LDS.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

// fp64 -> bits of a binary format with P significant bits, smallest quantum
// 2^QMIN and all-ones exponent INF: round to nearest, ties to even, subnormal
// results on the 2^QMIN grid, overflow to infinity.  Finite inputs only.
// bf16: P = 8, QMIN = -133, INF = 0x7F80; fp16: P = 11, QMIN = -24, INF = 0x7C00.
template <int P, int QMIN, uint32_t INF>
__device__ __forceinline__ uint16_t f64_to_bits_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  const int E = (int)(a >> 52);
  if (E == 0) return sign;  // zero or fp64 subnormal: far below half a quantum
  const int e = E - 1023;                          // value = S * 2^(e - 52)
  const uint64_t S = (a & 0x000FFFFFFFFFFFFFull) | (1ull << 52);
  const int q = e - (P - 1) > QMIN ? e - (P - 1) : QMIN;  // exponent of the last kept bit
  const int shift = q - e + 52;                    // >= 53 - P
  if (shift >= 60) return sign;                    // below half a quantum: rounds to zero
  uint64_t R = S >> shift;
  const uint64_t rem = S & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (R & 1))) ++R;
  if (R == 0) return sign;
  // value = R * 2^q with R <= 2^P (R >= 2^(P-1) unless q = QMIN)
  const int64_t bits = ((int64_t)(q - QMIN) << (P - 1)) + (int64_t)R;
  return (uint16_t)(sign | (bits >= (int64_t)INF ? INF : (uint32_t)bits));
}

__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  return f64_to_bits_rne<8, -133, 0x7F80u>(x);
}
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
  return f64_to_bits_rne<11, -24, 0x7C00u>(x);
}

// NC centres per group of 4 * NC weights, one lane per centre; 256 / NC groups
// per block.  SIGNMAG: u = |w|, levels to fp16, no scales; else u = w / absmax,
// levels to bf16 and the absmax written to scales.
template <int NC, bool SIGNMAG>
__global__ __launch_bounds__(256) void lloyd_fit_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                        int64_t k, int iters,
                                                        uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ levels) {
  constexpr int G = 4 * NC;      // weights per group
  constexpr int GB = 256 / NC;   // groups per block
  __shared__ double su[GB][G + 1];  // +1: consecutive groups start in different banks
  __shared__ double sc[GB][NC];
  __shared__ uint8_t sa[GB][G];
  const int tid = threadIdx.x, gl = tid / NC, j = tid % NC;
  const int64_t g = k / G, total = n * g;
  const int64_t t = (int64_t)blockIdx.x * GB + gl;
  const bool valid = t < total;

  double u[4] = {0.0, 0.0, 0.0, 0.0};
  if (valid) {
    const int64_t r = t / g, gi = t - r * g;
    const uint2 v = *reinterpret_cast<const uint2*>(w + r * k + gi * G + 4 * j);
    const uint32_t h[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (double)__uint_as_float(h[e] << 16);
  }
  double s = 0.0;
  bool zero = false;
  if constexpr (SIGNMAG) {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = fabs(u[e]);
  } else {
    // group absmax over the NC lanes (exact)
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fabs(u[e]) > s ? fabs(u[e]) : s;
#pragma unroll
    for (int o = NC / 2; o >= 1; o >>= 1) {
      const double other = __shfl_xor(s, o, NC);
      s = other > s ? other : s;
    }
    zero = !(s > 0.0);
    if (!zero) {
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = u[e] / s;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) su[gl][4 * j + e] = u[e];
  __syncthreads();

  // quantile start: stable rank of each element; ranks 4q + 2 become centres
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int me = 4 * j + e;
    int rank = 0;
    for (int i = 0; i < G; ++i) {
      const double v = su[gl][i];
      rank += (v < u[e] || (v == u[e] && i < me)) ? 1 : 0;
    }
    if ((rank & 3) == 2) sc[gl][rank >> 2] = u[e];
  }
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    double c[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) c[q] = sc[gl][q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int best = 0;
      double bd = fabs(u[e] - c[0]);
#pragma unroll
      for (int q = 1; q < NC; ++q) {
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
    for (int i = 0; i < G; ++i) {
      const bool mine = sa[gl][i] == j;
      const double v = su[gl][i];
      sum = mine ? sum + v : sum;
      cnt += mine ? 1 : 0;
    }
    if (cnt > 0) sc[gl][j] = sum / (double)cnt;
    __syncthreads();
  }

  if (valid) {
    if constexpr (SIGNMAG) {
      levels[t * NC + j] = f64_to_f16_rne(sc[gl][j]);
    } else {
      levels[t * NC + j] = zero ? (uint16_t)0 : f64_to_bf16_rne(sc[gl][j]);
      if (j == 0) scales[t] = f64_to_bf16_rne(s);  // s is a bf16 value: exact
    }
  }
}

}  // namespace

hipError_t launch_lut16_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* scales,
                            uint16_t* lut, int iters, hipStream_t stream) {
  const int64_t groups = n * (k / 64), per_block = 16;
  const int64_t blocks = (groups + per_block - 1) / per_block;
  lloyd_fit_kernel<16, false>
      <<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(w, n, k, iters, scales, lut);
  return hipGetLastError();
}

hipError_t launch_signmag8_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                               int iters, hipStream_t stream) {
  const int64_t groups = n * (k / 32), per_block = 32;
  const int64_t blocks = (groups + per_block - 1) / per_block;
  lloyd_fit_kernel<8, true>
      <<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(w, n, k, iters, nullptr, codebook);
  return hipGetLastError();
}

}  // namespace w4
