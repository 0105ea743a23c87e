// Per-group k-means fitting of the LUT codecs' tables (gfx950), and the
// int4-g32 page's warm start for the SIGNMAG8 magnitudes (further down).
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
#include <cmath>

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

// ---------------------------------------------------------------- warm start
// int4-g32 page, sections 1.2, 1.3 and 5.1: per group of 32 magnitudes a_i,
// 112 transforms f are tried; each maps the group into f-space, rounds it to
// 8 uniform levels q = rint(f / fmax * 7) (fmax = f(gmax)), maps the level
// grid (q / 7) * fmax back through the inverse of f and scores the group's
// squared error; the best transform's 8 levels start the Lloyd rounds.
// Candidates in increasing 8-bit parameter code (family << 7 | b_idx << 3 |
// beta_idx; the lowest code wins a tie):
//   bounded rational f(w) = w / (b + w^beta), b = b_rel * gmax, b_rel =
//     10^((5 i - 42) / 14) for i = 0..14, beta in kBetas; inverse: beta = 1
//     w = fd*b / (1 - fd), beta < 1 the root of w = fd*b + fd*w^beta;
//   tanh f(w) = tanh(w / b), b_rel in kBrelTanh; inverse w = b * atanh(fd).
// Everything in fp64; the error sum runs over the weights in element order.
constexpr int kCand = 112, kRat = 105, kWarmGroups = 2;  // groups per 256-thread block
struct BrelRat {
  double v[15];  // 10^((5 i - 42) / 14), computed on the host with the C library's pow
};
__constant__ double kBetas[7] = {0.50, 0.55, 0.65, 0.75, 0.85, 0.95, 1.00};
__constant__ double kBrelTanh[7] = {0.25, 0.4, 0.6, 0.85, 1.2, 1.8, 3.0};

// Root of g(w) = w - (fd*b + fd*w^beta), fd > 0, beta < 1.  g is negative at
// 0, convex, and increasing from below its root on, so Newton steps from any
// point right of the root fall monotonically onto it; 2 * gmax is right of it
// (f increases and fd <= f(gmax)).  Steps stop when they no longer move w down.
__device__ double rational_root(double fd, double b, double beta, double start) {
  double w = start;
  for (int it = 0; it < 200; ++it) {
    const double p = pow(w, beta);
    const double g = w - (fd * b + fd * p);
    if (!(g > 0.0)) break;
    const double d = 1.0 - fd * beta * (p / w);
    const double wn = w - g / d;
    if (!(wn < w)) break;
    w = wn;
  }
  return w;
}

__global__ __launch_bounds__(256) void warm_fit_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                       int64_t k, int iters,
                                                       BrelRat brel,
                                                       uint16_t* __restrict__ codebook,
                                                       uint8_t* __restrict__ params) {
  constexpr int G = 32, NC = 8, GB = kWarmGroups;
  __shared__ double sa[GB][G + 1];          // magnitudes
  __shared__ double spow[GB][6][G];         // a^beta for the six beta < 1
  __shared__ double sb[GB][kCand], sfmax[GB][kCand];
  __shared__ double slev[GB][kCand][NC];    // every candidate's 8 levels
  __shared__ double sgmax[GB];
  __shared__ double wbest[GB][2];           // per-wave argmin: error
  __shared__ int wbesti[GB][2];             //                 candidate
  __shared__ double sc[GB][NC];
  __shared__ uint8_t sasg[GB][G];
  const int tid = threadIdx.x;
  const int64_t g = k / G, total = n * g;
  const int64_t t0 = (int64_t)blockIdx.x * GB;

  // magnitudes (groups past the end read as zeros)
  if (tid < GB * G) {
    const int gl = tid / G, i = tid % G;
    const int64_t t = t0 + gl;
    double v = 0.0;
    if (t < total) {
      const int64_t r = t / g, gi = t - r * g;
      v = fabs((double)__uint_as_float((uint32_t)w[r * k + gi * G + i] << 16));
    }
    sa[gl][i] = v;
  }
  __syncthreads();
  if (tid < GB) {
    double m = 0.0;
    for (int i = 0; i < G; ++i) m = sa[tid][i] > m ? sa[tid][i] : m;
    sgmax[tid] = m;
  }
  // a^beta for beta < 1 (pow(0, beta) = 0)
  for (int e = tid; e < GB * 6 * G; e += 256) {
    const int gl = e / (6 * G), bi = (e / G) % 6, i = e % G;
    spow[gl][bi][i] = pow(sa[gl][i], kBetas[bi]);
  }
  __syncthreads();

  // per candidate: b and fmax = f(gmax)
  for (int e = tid; e < GB * kCand; e += 256) {
    const int gl = e / kCand, c = e % kCand;
    const double gm = sgmax[gl];
    if (!(gm > 0.0)) continue;
    double b, fmax;
    if (c < kRat) {
      const int bi = c / 7, ki = c % 7;
      b = brel.v[bi] * gm;
      const double gp = ki == 6 ? gm : pow(gm, kBetas[ki]);
      fmax = gm / (b + gp);
    } else {
      b = kBrelTanh[c - kRat] * gm;
      fmax = tanh(gm / b);
    }
    sb[gl][c] = b;
    sfmax[gl][c] = fmax;
  }
  __syncthreads();

  // levels: (q / 7) * fmax through the inverse, q = 1..7 (level 0 is 0).  The
  // beta < 1 roots (Newton) come first in the work order so that they spread
  // evenly over the threads.
  {
    constexpr int kHeavy = 15 * 6 * 7, kLight = (15 + 7) * 7;
    for (int e = tid; e < GB * (kHeavy + kLight); e += 256) {
      int gl, c, q;
      if (e < GB * kHeavy) {
        gl = e / kHeavy;
        const int r = e % kHeavy, ci = r / 7;
        c = (ci / 6) * 7 + ci % 6;
        q = r % 7 + 1;
      } else {
        const int e2 = e - GB * kHeavy;
        gl = e2 / kLight;
        const int r = e2 % kLight, ci = r / 7;
        c = ci < 15 ? ci * 7 + 6 : kRat + (ci - 15);
        q = r % 7 + 1;
      }
      const double gm = sgmax[gl];
      if (!(gm > 0.0)) continue;
      const double b = sb[gl][c];
      const double fd = ((double)q / 7.0) * sfmax[gl][c];
      double v;
      if (c >= kRat) {
        v = b * atanh(fd);
      } else if (c % 7 == 6) {
        v = (fd * b) / (1.0 - fd);
      } else {
        v = rational_root(fd, b, kBetas[c % 7], 2.0 * gm);
      }
      slev[gl][c][q] = v;
    }
    for (int e = tid; e < GB * kCand; e += 256) slev[e / kCand][e % kCand][0] = 0.0;
  }
  __syncthreads();

  // each candidate's squared error, then the argmin per group: candidate c of
  // group gl on thread gl * 128 + c (two waves per group)
  {
    const int gl = tid >> 7, c = tid & 127, wv = (tid >> 6) & 1;
    const double gm = sgmax[gl];
    double err = INFINITY;
    if (c < kCand && gm > 0.0) {
      const double b = sb[gl][c], fmax = sfmax[gl][c];
      const int ki = c < kRat ? c % 7 : -1;
      double acc = 0.0;
      for (int i = 0; i < G; ++i) {
        const double a = sa[gl][i];
        double f;
        if (ki < 0)
          f = tanh(a / b);
        else
          f = a / (b + (ki == 6 ? a : spow[gl][ki][i]));
        double qf = rint((f / fmax) * 7.0);
        qf = qf < 0.0 ? 0.0 : (qf > 7.0 ? 7.0 : qf);
        const double d = a - slev[gl][c][(int)qf];
        acc = acc + d * d;
      }
      err = acc;
    }
    // lowest error, lowest candidate on a tie
    int best = c;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double oe = __shfl_xor(err, o, 64);
      const int oc = __shfl_xor(best, o, 64);
      if (oe < err || (oe == err && oc < best)) {
        err = oe;
        best = oc;
      }
    }
    if ((tid & 63) == 0) {
      wbest[gl][wv] = err;
      wbesti[gl][wv] = best;
    }
  }
  __syncthreads();

  // Lloyd rounds from the winner's levels: 8 lanes per group, lane j holding
  // elements 4j .. 4j+3 and owning centre j
  const int lgl = tid / NC, j = tid % NC;
  const bool lloyd_lane = tid < GB * NC;
  int winner = 0;
  if (lloyd_lane) {
    const bool live = sgmax[lgl] > 0.0;
    const double e0 = wbest[lgl][0], e1 = wbest[lgl][1];
    winner = (e1 < e0) ? wbesti[lgl][1] : wbesti[lgl][0];
    if (!live || winner >= kCand) winner = -1;  // all-zero group (no finite error)
    sc[lgl][j] = winner >= 0 ? slev[lgl][winner][j] : 0.0;
  }
  __syncthreads();
  double u[4] = {0.0, 0.0, 0.0, 0.0};
  if (lloyd_lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = sa[lgl][4 * j + e];
  }
  for (int it = 0; it < iters; ++it) {
    if (lloyd_lane) {
      double c[NC];
#pragma unroll
      for (int q = 0; q < NC; ++q) c[q] = sc[lgl][q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int bq = 0;
        double bd = fabs(u[e] - c[0]);
#pragma unroll
        for (int q = 1; q < NC; ++q) {
          const double d = fabs(u[e] - c[q]);
          if (d < bd) {
            bd = d;
            bq = q;
          }
        }
        sasg[lgl][4 * j + e] = (uint8_t)bq;
      }
    }
    __syncthreads();
    if (lloyd_lane) {
      double sum = 0.0;
      int cnt = 0;
      for (int i = 0; i < G; ++i) {
        const bool mine = sasg[lgl][i] == j;
        const double v = sa[lgl][i];
        sum = mine ? sum + v : sum;
        cnt += mine ? 1 : 0;
      }
      if (cnt > 0) sc[lgl][j] = sum / (double)cnt;
    }
    __syncthreads();
  }

  if (lloyd_lane) {
    const int64_t t = t0 + lgl;
    if (t < total) {
      codebook[t * NC + j] = f64_to_f16_rne(sc[lgl][j]);
      if (params && j == 0) {
        uint8_t code = 0;
        if (winner >= kRat)
          code = (uint8_t)(128 | ((winner - kRat) << 3));
        else if (winner >= 0)
          code = (uint8_t)(((winner / 7) << 3) | (winner % 7));
        params[t] = code;
      }
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

hipError_t launch_signmag8_warm_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                                    uint8_t* params, int iters, hipStream_t stream) {
  BrelRat brel;
  for (int i = 0; i < 15; ++i) brel.v[i] = std::pow(10.0, (double)(5 * i - 42) / 14.0);
  const int64_t groups = n * (k / 32);
  const int64_t blocks = (groups + kWarmGroups - 1) / kWarmGroups;
  warm_fit_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(w, n, k, iters, brel,
                                                                     codebook, params);
  return hipGetLastError();
}

}  // namespace w4
