// Quantize + pack kernels (gfx950).
//
// DyadicGumbel page, sections 2.1-2.3 and 2.5: per group of 64 weights a bf16
// scale (the group absmax here) and for each weight the hard argmin over the
// 16 codes (scale/8)*(j-8); two 4-bit indices per byte, low nibble first.
// k-means page, section 1.2: nearest of the group's 16 LUT levels (a table
// per group, LUT16, or one table for the whole weight, LUT16S).
// int4-g32 page, sections 1.3 and 2: sign bit + nearest of 8 magnitudes.
//
// One thread handles 8 consecutive weights (one 16-byte load, one 4-byte
// packed store); a 64-weight group is 8 adjacent lanes, so the group absmax
// is three DPP steps inside the lane octet.  Rows hold whole groups (k is a
// multiple of 64), so the weight is processed as a flat array.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

// DPP lane moves (all lanes of an octet are active whenever these run).
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {  // lane i <-> 7 - i within 8 lanes
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x141, 0xF, 0xF, false));
}

__device__ __forceinline__ void unpack8(const u32x4& v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
}

// idx = #{t in 0..14 : w > (2t - 15) * s/16}: the number of midpoints between
// adjacent codes that lie strictly below w (ties go to the lower index).
// Every (2t-15)*s/16 is exact in fp32 (<= 12 significant bits, no overflow
// since it is below s), so each comparison is exact.
__device__ __forceinline__ uint32_t dyadic_idx_exact(float w, float s16) {
  uint32_t c = 0;
#pragma unroll
  for (int t = 0; t < 15; ++t) c += (w > (float)(2 * t - 15) * s16) ? 1u : 0u;
  return c;
}

// Same count, found from an estimate that is off by at most one and then
// checked against the two exact midpoints around it, in fp32 throughout:
// f0 = clamp(floor(8 w / s + 8), 0, 15) is the true count or one off; the
// midpoints below and above code f0 are (2 f0 - 17) s/16 and (2 f0 - 15) s/16
// (exact: at most 12 significant bits).  The one below code 0 exceeds the fp32
// range for the largest bf16 scales and becomes -inf (nothing lies below it,
// as it should); the one above is formed by one fma, (2 f0 - 17) s/16 + s/8,
// whose exact result is at most 15 s/16 in magnitude and so always finite.
__device__ __forceinline__ uint32_t dyadic_idx_fast(float w, float inv8, float s16, float s8) {
  float f0 = __builtin_floorf(__builtin_fmaf(w, inv8, 8.0f));
  f0 = __builtin_amdgcn_fmed3f(f0, 0.0f, 15.0f);
  const float t = __builtin_fmaf(f0, 2.0f, -17.0f);  // 2 f0 - 17, exact
  const float mlo = t * s16;                          // exact or -inf
  const float mhi = __builtin_fmaf(t, s16, s8);       // exact, finite
  const int i = (int)f0 - (w <= mlo ? 1 : 0) + (w > mhi ? 1 : 0);
  return (uint32_t)(i > 15 ? 15 : i);
}

__global__ __launch_bounds__(256) void quantize_dyadic_kernel(const u32x4* __restrict__ w,
                                                              uint32_t* __restrict__ packed,
                                                              uint16_t* __restrict__ scales,
                                                              int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = c < nchunks;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (live) v = __builtin_nontemporal_load(&w[c]);
  float f[8];
  unpack8(v, f);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(f[i]));
  a = __builtin_fmaxf(a, dpp_quad_xor1(a));
  a = __builtin_fmaxf(a, dpp_quad_xor2(a));
  a = __builtin_fmaxf(a, dpp_half_mirror(a));
  const float s = a;  // group absmax: a bf16 value, exact in fp32
  const float s16 = s * 0.0625f, s8 = s * 0.125f;
  uint32_t word = 0x88888888u;  // all-zero group: index 8 everywhere
  const bool tiny = s < 0x1p-120f;  // 8/s would overflow: use the direct count
  if (__builtin_expect(__any(tiny && s != 0.0f), 0)) {
    if (s != 0.0f) {
      word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= dyadic_idx_exact(f[i], s16) << (4 * i);
    }
  } else if (s != 0.0f) {
    const float inv8 = 8.0f / s;
    word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= dyadic_idx_fast(f[i], inv8, s16, s8) << (4 * i);
  }
  if (live) {
    packed[c] = word;
    if ((c & 7) == 0) scales[c >> 3] = (uint16_t)(__builtin_bit_cast(uint32_t, s) >> 16);
  }
}

// Nearest level, exactly: the lowest j minimising the exact |x - v_j|, for a
// value x and levels v_j that double holds exactly (bf16 weights, products of
// two bf16 numbers, fp16 magnitudes, +inf).  The distance rounded to double,
// fl(|x - v_j|), is monotone in the exact distance, so the first level at the
// smallest rounded distance is the answer unless another level shares that
// rounded distance (a true tie, or two distances that round alike because a
// level is far smaller or larger than x).  nearest_scan reports such a tie;
// nearest_settle then compares the tied levels' exact distances
// |h| + sgn(h) e, where h = fl(x - v_j) and e = (x - v_j) - h is the exact
// error of the subtraction (two-sum), and |h| is the same for all of them.
template <int NL>
__device__ __forceinline__ uint32_t nearest_scan(double x, const double (&v)[NL], double& dmin,
                                                 bool& tie) {
  double best = __builtin_fabs(x - v[0]);
  uint32_t bi = 0;
  bool t = false;
#pragma unroll
  for (int j = 1; j < NL; ++j) {
    const double d = __builtin_fabs(x - v[j]);
    t = d < best ? false : (t || d == best);
    if (d < best) {
      best = d;
      bi = (uint32_t)j;
    }
  }
  dmin = best;
  // every level +inf away: all tie exactly, and the lowest index is the answer
  tie = t && best != __builtin_inf();
  return bi;
}

template <int NL>
__device__ __forceinline__ uint32_t nearest_settle(double x, const double (&v)[NL], double dmin) {
  uint32_t bi = 0;
  double bk = __builtin_inf();
#pragma unroll
  for (int j = NL - 1; j >= 0; --j) {  // downwards: the lowest index wins equal keys
    const double h = x - v[j];
    const double bp = h - x;               // two-sum of x and -v_j
    const double ap = h - bp;
    const double e = (x - ap) + (-v[j] - bp);
    const double key = h < 0.0 ? -e : e;
    if (__builtin_fabs(h) == dmin && key <= bk) {
      bk = key;
      bi = (uint32_t)j;
    }
  }
  return bi;
}

// Levels in strictly increasing order whose midpoints (v_t + v_t+1) / 2 are
// exact in double (the sum's two-sum error is zero, which also rules out an
// infinite level): the lowest nearest level of x is then the number of
// midpoints strictly below x, since x lies nearer v_t+1 than v_t exactly
// when x > m_t, and x = m_t, a tie, keeps the lower index.  Fitted tables
// and magnitudes are sorted and distinct; any other table takes the scan.
template <int NL>
__device__ __forceinline__ bool exact_midpoints(const double (&v)[NL], double (&mid)[NL - 1]) {
  bool ok = true;
#pragma unroll
  for (int t = 0; t < NL - 1; ++t) {
    const double a = v[t], b = v[t + 1];
    const double sum = a + b;
    const double bp = sum - a;
    const double ap = sum - bp;
    const double e = (a - ap) + (b - bp);
    ok = ok && a < b && e == 0.0;
    mid[t] = sum * 0.5;
  }
  return ok;
}

// Eight weights against NL levels: the packed word of their indices (plus
// the sign bits for SIGNMAG8, where x = |w|).  Lanes whose levels qualify
// count midpoints; a wave with any other lane also runs the scan for those,
// and settles ties only if one of its lanes has one.
template <int NL, bool SIGNMAG>
__device__ __forceinline__ uint32_t nearest8(const float (&f)[8], const double (&v)[NL],
                                             const double (&mid)[NL - 1], bool counted) {
  uint32_t idx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double x = SIGNMAG ? (double)__builtin_fabsf(f[i]) : (double)f[i];
    uint32_t n = 0;
#pragma unroll
    for (int t = 0; t < NL - 1; ++t) n += x > mid[t] ? 1u : 0u;
    idx[i] = n;
  }
  if (__builtin_expect(__any(!counted), 0)) {
    double dmin[8];
    bool any_tie = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double x = SIGNMAG ? (double)__builtin_fabsf(f[i]) : (double)f[i];
      bool t;
      const uint32_t j = nearest_scan<NL>(x, v, dmin[i], t);
      if (!counted) idx[i] = j;
      any_tie = any_tie || (t && !counted);
    }
    if (__builtin_expect(__any(any_tie), 0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double x = SIGNMAG ? (double)__builtin_fabsf(f[i]) : (double)f[i];
        if (!counted && dmin[i] != __builtin_inf()) idx[i] = nearest_settle<NL>(x, v, dmin[i]);
      }
    }
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sign = (SIGNMAG && f[i] < 0.0f) ? 8u : 0u;
    word |= (sign | idx[i]) << (4 * i);
  }
  return word;
}

// LUT16 / LUT16S: levels v_j = s * L_j (exact in double); index = the exact
// nearest level.  shared: one table for every group (LUT16S).  One thread
// per group of 64: the levels and their midpoints are set up once for the
// group's eight chunks, whose loads are all issued first (cached loads: the
// lanes' chunks interleave within lines that the next loads reuse).
__global__ __launch_bounds__(256) void quantize_lut16_kernel(const u32x4* __restrict__ w,
                                                             uint32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             const u32x4* __restrict__ lut,
                                                             int64_t ngroups, int shared) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  const int64_t gt = shared ? 0 : g;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = w[8 * g + i];
  const double s = (double)bf16_bits_to_f32(scales[g]);
  const u32x4 l0 = lut[2 * gt], l1 = lut[2 * gt + 1];
  const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
  double lv[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lv[2 * i] = (double)bf16_bits_to_f32(lw[i] & 0xFFFFu) * s;
    lv[2 * i + 1] = (double)__builtin_bit_cast(float, lw[i] & 0xFFFF0000u) * s;
  }
  double mid[15];
  const bool counted = exact_midpoints<16>(lv, mid);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[8];
    unpack8(v[i], f);
    packed[8 * g + i] = nearest8<16, false>(f, lv, mid, counted);
  }
}

// SIGNMAG8: nibble = (w < 0) << 3 | the exact nearest magnitude to |w|.  One
// thread per group of 32 (four chunks), as for LUT16.
__global__ __launch_bounds__(256) void quantize_signmag8_kernel(const u32x4* __restrict__ w,
                                                                uint32_t* __restrict__ packed,
                                                                const u32x4* __restrict__ cb,
                                                                int64_t ngroups) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ngroups) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = w[4 * g + i];
  const u32x4 m = cb[g];
  const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
  double mv[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 h = __builtin_bit_cast(f16x2, mw[i]);
    mv[2 * i] = (double)(float)h.x;
    mv[2 * i + 1] = (double)(float)h.y;
  }
  double mid[7];
  const bool counted = exact_midpoints<8>(mv, mid);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[8];
    unpack8(v[i], f);
    packed[4 * g + i] = nearest8<8, true>(f, mv, mid, counted);
  }
}

// Bit of a run's 32-bit high-bit word that holds weight i (0..31) of the run
// (the layout w4_device.h's dyadic5_msb reads).
__device__ __forceinline__ constexpr int dyadic5_msb_bit(int i) {
  constexpr int P[8] = {4, 8, 4, 8, 20, 24, 20, 24};
  constexpr int A[8] = {-4, -3, -2, -1, 4, 5, 6, 7};
  return P[i % 8] + A[2 * (i / 8) + ((i % 8) % 4 >= 2 ? 1 : 0)];
}

// DYADIC5: one thread per run of 32 weights (two threads per 64-group).
// Group width b in {3, 4, 5}, half = 2^(b-1): the b-bit index is the number
// of midpoints m_t = (2t + 1 - 2 half) * s / (2 half), t = 0 .. 2 half - 2,
// below w (strictly: a weight on a midpoint takes the lower code), found by a
// binary search; every m_t is exact in fp32 (an odd integer below 64 times a
// power-of-two fraction of a bf16 scale).  Stored as j5 = index << (5 - b).
__global__ __launch_bounds__(256) void quantize_dyadic5_kernel(const u32x4* __restrict__ w,
                                                               const uint8_t* __restrict__ widths,
                                                               u32x4* __restrict__ packed,
                                                               uint32_t* __restrict__ msb,
                                                               uint16_t* __restrict__ scales,
                                                               int64_t nruns) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = c < nruns;
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = __builtin_nontemporal_load(&w[4 * c + i]);
    unpack8(v, &f[8 * i]);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(f[i]));
  a = __builtin_fmaxf(a, __shfl_xor(a, 1));  // the other half of the 64-group
  const int64_t g = c >> 1;
  int b = 5;
  if (live && widths) {
    const int wb = widths[g];
    b = (wb == 3 || wb == 4) ? wb : 5;
  }
  const int half = 1 << (b - 1), top = 2 * half - 1;  // top = number of midpoints
  const float step2 = a * (0.5f / (float)half);        // s / (2 half), exact
  uint32_t words[4] = {0u, 0u, 0u, 0u}, M = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    int cnt = 0;
#pragma unroll
    for (int bit = 16; bit >= 1; bit >>= 1) {
      const int t = cnt + bit - 1;  // candidate midpoint index
      if (cnt + bit <= top && f[i] > (float)(2 * t + 1 - 2 * half) * step2) cnt += bit;
    }
    if (a == 0.0f) cnt = half;  // all-zero group: the zero code
    const uint32_t j5 = (uint32_t)cnt << (5 - b);
    words[i / 8] |= (j5 & 15u) << (4 * (i % 8));
    M |= (j5 >> 4) << dyadic5_msb_bit(i);
  }
  if (live) {
    packed[c] = (u32x4){words[0], words[1], words[2], words[3]};
    msb[c] = M;
    if ((c & 1) == 0) scales[g] = (uint16_t)(__builtin_bit_cast(uint32_t, a) >> 16);
  }
}

// W4_LUT16S_IL records from the planar LUT16S arrays: per row and 256-k
// block, chunks 0-7 are the block's 128 packed bytes and chunk 8 holds its
// four bf16 scales followed by 8 zero bytes.  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void lut16s_interleave_kernel(const u32x4* __restrict__ packed,
                                                                const uint16_t* __restrict__ scales,
                                                                u32x4* __restrict__ out,
                                                                int64_t nchunks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nchunks) return;
  const int64_t rb = t / 9, c = t % 9;  // record (row-major over rows and 256-k blocks), chunk
  u32x4 v;
  if (c < 8) {
    v = packed[rb * 8 + c];
  } else {
    const uint16_t* sc = scales + rb * 4;
    v = (u32x4){(uint32_t)sc[0] | ((uint32_t)sc[1] << 16), (uint32_t)sc[2] | ((uint32_t)sc[3] << 16),
                0u, 0u};
  }
  out[t] = v;
}

}  // namespace

hipError_t launch_lut16s_interleave(int64_t n, int64_t k, const uint8_t* packed,
                                    const uint16_t* scales, uint8_t* out, hipStream_t stream) {
  const int64_t nchunks = n * (k / 256) * 9;
  const int64_t blocks = (nchunks + 255) / 256;
  lut16s_interleave_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const u32x4*>(packed), scales, reinterpret_cast<u32x4*>(out), nchunks);
  return hipGetLastError();
}

hipError_t launch_quantize_dyadic5(int64_t n, int64_t k, const uint16_t* w, const uint8_t* widths,
                                   uint8_t* packed, uint8_t* msb, uint16_t* scales,
                                   hipStream_t stream) {
  const int64_t nruns = n * k / 32;
  const int64_t blocks = (nruns + 255) / 256;
  quantize_dyadic5_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const u32x4*>(w), widths, reinterpret_cast<u32x4*>(packed),
      reinterpret_cast<uint32_t*>(msb), scales, nruns);
  return hipGetLastError();
}

hipError_t launch_quantize(int codec, int64_t n, int64_t k, const uint16_t* w, uint8_t* packed,
                           uint16_t* scales, const uint16_t* codebook, hipStream_t stream) {
  const int64_t nchunks = n * k / 8;
  const int64_t blocks = (nchunks + 255) / 256;
  const auto* wv = reinterpret_cast<const u32x4*>(w);
  auto* pk = reinterpret_cast<uint32_t*>(packed);
  if (codec == 0)
    quantize_dyadic_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(wv, pk, scales, nchunks);
  else if (codec == 1 || codec == 3)
    quantize_lut16_kernel<<<dim3((uint32_t)((nchunks / 8 + 255) / 256)), dim3(256), 0, stream>>>(
        wv, pk, scales, reinterpret_cast<const u32x4*>(codebook), nchunks / 8, codec == 3);
  else
    quantize_signmag8_kernel<<<dim3((uint32_t)((nchunks / 4 + 255) / 256)), dim3(256), 0, stream>>>(
        wv, pk, reinterpret_cast<const u32x4*>(codebook), nchunks / 4);
  return hipGetLastError();
}

}  // namespace w4
