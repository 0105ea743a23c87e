// Unpack + rebuild to a dense weight (gfx950).
//
// DyadicGumbel page, section 2.5: the unpack kernel loads a packed byte,
// splits the nibbles, looks up the step and rebuilds bf16 (there: 1024
// elements per program, one launch per layer).  k-means page, section 2.2:
// decode by table lookup (LUT16, and LUT16S with one table for every group).
// int4-g32 page, section 2: (level table, sign) per group -> dense fp16 weight.
//
// One thread rebuilds 16 packed bytes (32 weights): a 16-byte load and four
// 16-byte stores, so a wave moves 1 KiB in and 4 KiB out with full lines.
// 32 weights are half a 64-group (one scale / one LUT) or one 32-group.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {
namespace {

__global__ __launch_bounds__(256) void dequant_dyadic_kernel(const u32x4* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             u32x4* __restrict__ out,
                                                             int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = c < nchunks;
  u32x4 p = {0u, 0u, 0u, 0u};
  uint32_t sb = 0;
  if (live) {
    p = __builtin_nontemporal_load(&packed[c]);
    sb = scales[c >> 1];
  }
  const DyadicScale d = dyadic_scale(sb);
  const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, mg = kMagic;
  const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
  u32x4 o[4];
  if (__builtin_expect(__any(dyadic_scale_is_wide(sb)), 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = sigma_to_natural(dyadic_rebuild_wide(pw[i], d, m0, m1, mg));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = sigma_to_natural(dyadic_rebuild(pw[i], d, m0, m1, mg));
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(o[i], &out[4 * c + i]);
  }
}

// shared: one table for every group (LUT16S)
__global__ __launch_bounds__(256) void dequant_lut16_kernel(const u32x4* __restrict__ packed,
                                                            const uint16_t* __restrict__ scales,
                                                            const u32x4* __restrict__ lut,
                                                            u32x4* __restrict__ out,
                                                            int64_t nchunks, int shared) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int64_t g = c >> 1, gt = shared ? 0 : g;
  const u32x4 p = __builtin_nontemporal_load(&packed[c]);
  const Lut16Table t = lut16_table(scales[g], lut[2 * gt], lut[2 * gt + 1]);
  const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_nontemporal_store(sigma_to_natural(lut16_rebuild(pw[i], t)), &out[4 * c + i]);
}

// fp16 output: bytes of +-M[mag] straight from an 8-entry byte-plane table.
__global__ __launch_bounds__(256) void dequant_signmag8_kernel(const u32x4* __restrict__ packed,
                                                               const u32x4* __restrict__ cb,
                                                               u32x4* __restrict__ out,
                                                               int64_t nchunks) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const u32x4 p = __builtin_nontemporal_load(&packed[c]);
  const u32x4 m = cb[c];
  // byte planes of the 8 fp16 magnitudes
  const uint32_t tl0 = perm(m.y, m.x, 0x06040200u), tl1 = perm(m.w, m.z, 0x06040200u);
  const uint32_t th0 = perm(m.y, m.x, 0x07050301u), th1 = perm(m.w, m.z, 0x07050301u);
  const uint32_t pw[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = pw[i];
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
    __builtin_nontemporal_store(o, &out[4 * c + i]);
  }
}

// +0.0f the optimiser cannot see through (keeps the fma form of the rebuild)
__device__ __forceinline__ float opaque_pz() {
  uint32_t v = 0u;
  asm volatile("" : "+v"(v));
  return __builtin_bit_cast(float, v);
}

// DYADIC5: one thread per run of 32 weights: 16 packed bytes, the run's
// high-bit word and the group scale -> four 16-byte stores.
__global__ __launch_bounds__(256) void dequant_dyadic5_kernel(const u32x4* __restrict__ packed,
                                                              const uint32_t* __restrict__ msb,
                                                              const uint16_t* __restrict__ scales,
                                                              u32x4* __restrict__ out,
                                                              int64_t nruns) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nruns) return;
  const u32x4 p = __builtin_nontemporal_load(&packed[c]);
  const uint32_t M = msb[c];
  const Dyadic5Scale d = dyadic5_scale(scales[c >> 1]);
  const float pz = opaque_pz();
  uint32_t e0, e1;
  dyadic5_msb<0>(M, e0, e1);
  __builtin_nontemporal_store(sigma_to_natural(dyadic5_rebuild(p.x, e0, e1, d, pz)), &out[4 * c]);
  dyadic5_msb<1>(M, e0, e1);
  __builtin_nontemporal_store(sigma_to_natural(dyadic5_rebuild(p.y, e0, e1, d, pz)), &out[4 * c + 1]);
  dyadic5_msb<2>(M, e0, e1);
  __builtin_nontemporal_store(sigma_to_natural(dyadic5_rebuild(p.z, e0, e1, d, pz)), &out[4 * c + 2]);
  dyadic5_msb<3>(M, e0, e1);
  __builtin_nontemporal_store(sigma_to_natural(dyadic5_rebuild(p.w, e0, e1, d, pz)), &out[4 * c + 3]);
}

}  // namespace

hipError_t launch_dequant(int codec, int64_t n, int64_t k, const uint8_t* packed,
                          const uint16_t* scales, const uint16_t* codebook, void* out,
                          hipStream_t stream) {
  const int64_t nchunks = n * k / 32;
  const int64_t blocks = (nchunks + 255) / 256;
  const auto* pk = reinterpret_cast<const u32x4*>(packed);
  auto* o = reinterpret_cast<u32x4*>(out);
  if (codec == 0)
    dequant_dyadic_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(pk, scales, o, nchunks);
  else if (codec == 1 || codec == 3)
    dequant_lut16_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, scales, reinterpret_cast<const u32x4*>(codebook), o, nchunks, codec == 3);
  else if (codec == 4)
    dequant_dyadic5_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, reinterpret_cast<const uint32_t*>(codebook), scales, o, nchunks);  // chunk = run of 32
  else
    dequant_signmag8_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
        pk, reinterpret_cast<const u32x4*>(codebook), o, nchunks);
  return hipGetLastError();
}

}  // namespace w4
