// Unpack + rebuild to a dense weight (gfx950).
//
// DyadicGumbel page, section 2.5: the unpack kernel loads a packed byte,
// splits the nibbles, looks up the step and rebuilds bf16 (there: 1024
// elements per program, one launch per layer).  k-means page, section 2.2:
// decode by table lookup (LUT16, and LUT16S with one table for every group).
// int4-g32 page, section 2: (level table, sign) per group -> dense fp16 weight.
//
// One thread rebuilds four packed dwords (8 weights each), 64 dwords apart,
// so that each of a wave's loads and stores covers whole lines (below).
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

// Packed dword d of the flat weight holds weights 8d .. 8d+7 (one 16-byte
// output chunk).  A wave takes 256 consecutive dwords; lane l rebuilds dwords
// 64 i + l (i = 0..3), so every load instruction reads 256 contiguous bytes
// and every store instruction writes 1 KiB of whole 128-byte lines.  (Four
// chunks of one lane side by side would make each store instruction write a
// quarter of every line it touches; with streaming stores the partial lines
// go to memory one by one, at half the bandwidth or less.)
__device__ __forceinline__ int64_t wave_dword(int i) {
  return ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256 + 64 * i + (threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void dequant_dyadic_kernel(const uint32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             u32x4* __restrict__ out, int64_t ndw) {
  uint32_t pw[4], sb[4];
  bool wide = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d = wave_dword(i);
    const bool live = d < ndw;
    pw[i] = live ? __builtin_nontemporal_load(&packed[d]) : 0u;
    sb[i] = live ? scales[d >> 3] : 0u;  // 8 dwords per group of 64
    wide |= dyadic_scale_is_wide(sb[i]);
  }
  const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, mg = kMagic;
  u32x4 o[4];
  if (__builtin_expect(__any(wide), 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = sigma_to_natural(dyadic_rebuild_wide(pw[i], dyadic_scale(sb[i]), m0, m1, mg));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = sigma_to_natural(dyadic_rebuild(pw[i], dyadic_scale(sb[i]), m0, m1, mg));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d = wave_dword(i);
    if (d < ndw) __builtin_nontemporal_store(o[i], &out[d]);
  }
}

// shared: one table for every group (LUT16S)
__global__ __launch_bounds__(256) void dequant_lut16_kernel(const uint32_t* __restrict__ packed,
                                                            const uint16_t* __restrict__ scales,
                                                            const u32x4* __restrict__ lut,
                                                            u32x4* __restrict__ out, int64_t ndw,
                                                            int shared) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d = wave_dword(i);
    if (d < ndw) {
      const int64_t g = d >> 3, gt = shared ? 0 : g;
      const uint32_t p = __builtin_nontemporal_load(&packed[d]);
      const Lut16Table t = lut16_table(scales[g], lut[2 * gt], lut[2 * gt + 1]);
      __builtin_nontemporal_store(sigma_to_natural(lut16_rebuild(p, t)), &out[d]);
    }
  }
}

// fp16 output: bytes of +-M[mag] straight from an 8-entry byte-plane table.
__global__ __launch_bounds__(256) void dequant_signmag8_kernel(const uint32_t* __restrict__ packed,
                                                               const u32x4* __restrict__ cb,
                                                               u32x4* __restrict__ out,
                                                               int64_t ndw) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d = wave_dword(i);
    if (d >= ndw) continue;
    const uint32_t w = __builtin_nontemporal_load(&packed[d]);
    const u32x4 m = cb[d >> 2];  // 4 dwords per group of 32
    // byte planes of the 8 fp16 magnitudes
    const uint32_t tl0 = perm(m.y, m.x, 0x06040200u), tl1 = perm(m.w, m.z, 0x06040200u);
    const uint32_t th0 = perm(m.y, m.x, 0x07050301u), th1 = perm(m.w, m.z, 0x07050301u);
    const uint32_t q = w & 0x07070707u, r = (w >> 4) & 0x07070707u;
    const uint32_t ql = perm(tl1, tl0, q), qh = perm(th1, th0, q) ^ ((w << 4) & 0x80808080u);
    const uint32_t rl = perm(tl1, tl0, r), rh = perm(th1, th0, r) ^ (w & 0x80808080u);
    const uint32_t q0 = perm(qh, ql, 0x05010400u);  // (k0, k2)
    const uint32_t q1 = perm(qh, ql, 0x07030602u);  // (k4, k6)
    const uint32_t r0 = perm(rh, rl, 0x05010400u);  // (k1, k3)
    const uint32_t r1 = perm(rh, rl, 0x07030602u);  // (k5, k7)
    u32x4 o;
    o.x = perm(r0, q0, 0x05040100u);  // (k0, k1)
    o.y = perm(r0, q0, 0x07060302u);  // (k2, k3)
    o.z = perm(r1, q1, 0x05040100u);  // (k4, k5)
    o.w = perm(r1, q1, 0x07060302u);  // (k6, k7)
    __builtin_nontemporal_store(o, &out[d]);
  }
}

// +0.0f the optimiser cannot see through (keeps the fma form of the rebuild)
__device__ __forceinline__ float opaque_pz() {
  uint32_t v = 0u;
  asm volatile("" : "+v"(v));
  return __builtin_bit_cast(float, v);
}

// DYADIC5: dword d is dword d % 4 of the run of 32 weights d / 4, whose
// high-bit word is msb[d / 4]; d % 4 is the lane's own lane % 4 for every i.
__global__ __launch_bounds__(256) void dequant_dyadic5_kernel(const uint32_t* __restrict__ packed,
                                                              const uint32_t* __restrict__ msb,
                                                              const uint16_t* __restrict__ scales,
                                                              u32x4* __restrict__ out,
                                                              int64_t ndw) {
  const float pz = opaque_pz();
  const int D = threadIdx.x & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t d = wave_dword(i);
    if (d >= ndw) continue;
    const uint32_t p = __builtin_nontemporal_load(&packed[d]);
    const uint32_t M = msb[d >> 2];
    const uint32_t sb = scales[d >> 3];
    const Dyadic5Scale sc = dyadic5_scale(sb);
    uint32_t e0, e1;
    if (D == 0)
      dyadic5_msb<0>(M, e0, e1);
    else if (D == 1)
      dyadic5_msb<1>(M, e0, e1);
    else if (D == 2)
      dyadic5_msb<2>(M, e0, e1);
    else
      dyadic5_msb<3>(M, e0, e1);
    u32x4 v;
    if (__builtin_expect(__any(dyadic5_scale_is_wide(sb)), 0))
      v = dyadic5_rebuild(p, e0, e1, sc, pz);
    else
      v = dyadic5_rebuild_fma(p, e0, e1, sc);
    __builtin_nontemporal_store(sigma_to_natural(v), &out[d]);
  }
}

}  // namespace

hipError_t launch_dequant(int codec, int64_t n, int64_t k, const uint8_t* packed,
                          const uint16_t* scales, const uint16_t* codebook, void* out,
                          hipStream_t stream) {
  const int64_t ndw = n * k / 8;                 // packed dwords = 16-byte output chunks
  const int64_t blocks = (ndw + 1023) / 1024;   // 4 waves x 256 dwords
  const auto* pk = reinterpret_cast<const uint32_t*>(packed);
  auto* o = reinterpret_cast<u32x4*>(out);
  if (codec == 0)
    dequant_dyadic_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(pk, scales, o, ndw);
  else if (codec == 1 || codec == 3)
    dequant_lut16_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, scales, reinterpret_cast<const u32x4*>(codebook), o, ndw, codec == 3);
  else if (codec == 4)
    dequant_dyadic5_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, reinterpret_cast<const uint32_t*>(codebook), scales, o, ndw);
  else
    dequant_signmag8_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, reinterpret_cast<const u32x4*>(codebook), o, ndw);
  return hipGetLastError();
}

}  // namespace w4
