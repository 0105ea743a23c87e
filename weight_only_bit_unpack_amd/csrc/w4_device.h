// Device-side building blocks shared by the gfx950 kernels of libw4.
//
// Rebuild of packed nibbles into MFMA B operands.  A lane rebuilds one dword
// of packed weights (8 consecutive k of one row) into 8 bf16 values held as 4
// VGPRs (one bf16x8 MFMA operand).  The values come out in the slot order
//     SIGMA = { k0, k4, k1, k5, k2, k6, k3, k7 }
// because that order falls out of two masks per 16-bit half: the nibbles of
// k0 and k4 sit in bits 0-3 of the two halves of the dword, those of k1 and
// k5 in bits 4-7.  The activation operand is staged in the same order, so the
// MFMA's sum over k is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp16 bit pattern 0x6400 is 1024.0: OR-ing a nibble into bits 0-3 of a half
// gives 1024 + n, into bits 4-7 gives 1024 + 16 n -- both exact in fp16.
constexpr uint32_t kMagic = 0x64006400u;

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// byte permute: result byte i = byte sel[i] of the 8-byte value {hi, lo}
// (selector 0..3 -> lo, 4..7 -> hi).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;  // v_cvt_pk_bf16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------- DYADIC
// w_hat = RNE_bf16(s8 * (n - 8)), s8 = scale / 8.
// Fast form: one fma per value on the fp16 magic number h:
//   h = 1024 + n      : fma(h, s8,      -1032 * s8) = s8 * (n - 8)
//   h = 1024 + 16 n   : fma(h, s8 / 16, -72   * s8) = s8 * (n - 8)
// The exact result has at most 11 significant bits, so the single rounding of
// the fma is exact, and the conversion to bf16 is the one RNE.  The constants
// -1032*s8 and -72*s8 are exact unless they overflow, i.e. for |s8| >= 2^117;
// scales that large take the wide form below (d = h - 1032 in fp16, exact).
struct DyadicScale {
  float s8, c1, s8_16, c2;
};

__device__ __forceinline__ DyadicScale dyadic_scale(uint32_t sbits) {
  DyadicScale d;
  d.s8 = bf16_bits_to_f32(sbits) * 0.125f;
  d.c1 = -1032.0f * d.s8;
  d.s8_16 = d.s8 * 0.0625f;
  d.c2 = -72.0f * d.s8;
  return d;
}

__device__ __forceinline__ bool dyadic_scale_is_wide(uint32_t sbits) {
  // |s8| >= 2^117  <=>  |scale| >= 2^120  <=>  bf16 exponent field >= 127 + 120
  return ((sbits >> 7) & 0xFFu) >= 247u;
}

__device__ __forceinline__ uint32_t fma_pair(uint32_t h2, float s, float c) {
  f16x2 h = __builtin_bit_cast(f16x2, h2);
  return cvt_pk_bf16(__builtin_fmaf((float)h.x, s, c), __builtin_fmaf((float)h.y, s, c));
}

// +0.0f that the optimiser cannot fold: fma(d, s, +0) is d * s for every
// nonzero product and +0 for an exact zero of either sign ((-0) + (+0) = +0).
__device__ __forceinline__ float hidden_pos_zero() {
  uint32_t z = 0u;
  asm volatile("" : "+v"(z));
  return __builtin_bit_cast(float, z);
}

__device__ __forceinline__ uint32_t wide_pair(uint32_t h2, float off, float s, float pz) {
  f16x2 h = __builtin_bit_cast(f16x2, h2);
  f16x2 o = {(_Float16)off, (_Float16)off};
  f16x2 d = h - o;  // exact: small integers (times 16); code 8 gives +0
  // the +0 addend keeps code 8 at +0 for a negative scale as well
  return cvt_pk_bf16(__builtin_fmaf((float)d.x, s, pz), __builtin_fmaf((float)d.y, s, pz));
}

// Branch-free form valid for every scale: d = h - off in fp16 (exact small
// integers: n - 8, or 16 (n - 8) for the high nibbles), then one fp32
// product per value (v_fma_mix with a -0 addend leaves the product as is) and
// the one RNE.  One VALU per pair more than the fast form; used where a
// uniform branch on the scale would split the instruction stream.
// The addend nz is -0.0f hidden from the optimiser (see dyadic_rebuild_any):
// fma(d, s, -0) is d * s for every d and s, and the fma keeps the fp16 operand
// inside v_fma_mix instead of a separate conversion.
__device__ __forceinline__ uint32_t sub_mul_pair(uint32_t h2, uint32_t off2, float s, float nz) {
  const f16x2 d = __builtin_bit_cast(f16x2, h2) - __builtin_bit_cast(f16x2, off2);
  return cvt_pk_bf16(__builtin_fmaf((float)d.x, s, nz), __builtin_fmaf((float)d.y, s, nz));
}

// One packed dword -> 8 bf16 values in SIGMA order, any scale.
// nz: -0.0f passed through an opaque register by the caller.
__device__ __forceinline__ u32x4 dyadic_rebuild_any(uint32_t p, const DyadicScale& d, uint32_t m0,
                                                    uint32_t m1, uint32_t mg, float nz) {
  const uint32_t q = p >> 8;
  const uint32_t o1 = 0x64086408u;  // fp16 1032 twice
  const uint32_t o2 = 0x64806480u;  // fp16 1152 twice
  u32x4 r;
  r.x = sub_mul_pair(and_or(p, m0, mg), o1, d.s8, nz);
  r.y = sub_mul_pair(and_or(p, m1, mg), o2, d.s8_16, nz);
  r.z = sub_mul_pair(and_or(q, m0, mg), o1, d.s8, nz);
  r.w = sub_mul_pair(and_or(q, m1, mg), o2, d.s8_16, nz);
  return r;
}

// One packed dword -> 8 bf16 values in SIGMA order.
__device__ __forceinline__ u32x4 dyadic_rebuild(uint32_t p, const DyadicScale& d, uint32_t m0,
                                                uint32_t m1, uint32_t mg) {
  const uint32_t q = p >> 8;
  const uint32_t v0 = and_or(p, m0, mg);  // k0, k4 : 1024 + n
  const uint32_t v1 = and_or(p, m1, mg);  // k1, k5 : 1024 + 16n
  const uint32_t v2 = and_or(q, m0, mg);  // k2, k6
  const uint32_t v3 = and_or(q, m1, mg);  // k3, k7
  u32x4 r;
  r.x = fma_pair(v0, d.s8, d.c1);
  r.y = fma_pair(v1, d.s8_16, d.c2);
  r.z = fma_pair(v2, d.s8, d.c1);
  r.w = fma_pair(v3, d.s8_16, d.c2);
  return r;
}

__device__ __forceinline__ u32x4 dyadic_rebuild_wide(uint32_t p, const DyadicScale& d, uint32_t m0,
                                                     uint32_t m1, uint32_t mg) {
  const uint32_t q = p >> 8;
  const float pz = hidden_pos_zero();
  u32x4 r;
  r.x = wide_pair(and_or(p, m0, mg), 1032.0f, d.s8, pz);
  r.y = wide_pair(and_or(p, m1, mg), 1152.0f, d.s8_16, pz);
  r.z = wide_pair(and_or(q, m0, mg), 1032.0f, d.s8, pz);
  r.w = wide_pair(and_or(q, m1, mg), 1152.0f, d.s8_16, pz);
  return r;
}

// ---------------------------------------------------------------- table lookups
// A 16-entry byte table lives in 4 dwords t0..t3 (entry j = byte j%4 of t[j/4]).
// n holds four 4-bit indices, one per byte.  Entries 0-7 come from {t1,t0},
// entries 8-15 from {t3,t2} (index xor 8), and `merge` picks per byte.
__device__ __forceinline__ uint32_t lookup16(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3,
                                             uint32_t n, uint32_t nx8, uint32_t merge) {
  const uint32_t a = perm(t1, t0, n);
  const uint32_t b = perm(t3, t2, nx8);
  return perm(b, a, merge);
}

// merge selector for 4 indices whose bit 3 sits at bit (8i + 3) of `x`:
// byte i selects byte i of the low-entry result, or byte i + 4 of the high one.
__device__ __forceinline__ uint32_t merge_sel(uint32_t x_shifted_by_1) {
  return and_or(x_shifted_by_1, 0x04040404u, 0x03020100u);
}

// ---------------------------------------------------------------- DYADIC5
// w_hat = RNE_bf16((s/16) * (j - 16)), j = nibble | high bit << 4.
// The high bit becomes one more mantissa bit of the fp16 magic number:
//   nibble in bits 0-3, high bit in bit 4:  h = 1024 + j,       (h - 1040) * s/16
//   nibble in bits 4-7, high bit in bit 8:  h = 1024 + 16 j,    (h - 1280) * s/256
// h - 1040 and h - 1280 are exact small integers (times 16) in fp16, the
// products are exact in fp32 for every bf16 scale, and the conversion is the
// one RNE.  The addend pz is +0.0f hidden from the optimiser: an exact zero
// product then comes out +0 even for a zero scale.
// With the offsets folded into one fma, (h - 1040) s/16 = fma(h, s/16, -1040 s/16)
// and (h - 1280) s/256 = fma(h, s/256, -1280 s/256): the constants are exact
// (at most 15 significant bits) unless they overflow, which needs a scale of
// 2^120 or more (dyadic5_scale_is_wide); the fma's exact result has at most
// 13 significant bits, so its one rounding is exact, and an exact zero comes
// out +0 (x + (-x)).  Wide scales take the subtract-then-multiply form.
struct Dyadic5Scale {
  float s16, s256, c1, c2;
};

__device__ __forceinline__ Dyadic5Scale dyadic5_scale(uint32_t sbits) {
  Dyadic5Scale d;
  d.s16 = bf16_bits_to_f32(sbits) * 0.0625f;
  d.s256 = d.s16 * 0.0625f;
  d.c1 = -1040.0f * d.s16;
  d.c2 = -1280.0f * d.s256;
  return d;
}

__device__ __forceinline__ bool dyadic5_scale_is_wide(uint32_t sbits) {
  return ((sbits >> 7) & 0xFFu) >= 247u;  // |scale| >= 2^120
}

// High bits of packed dword D (0..3) of a run of 32 weights, from the run's
// word M: the first two value pairs take M shifted by A[2D], the last two by
// A[2D + 1], A = {-4, -3, -2, -1, 4, 5, 6, 7} (negative: left shift); the
// pairs' high bits then sit at bits (4, 20) and (8, 24).
template <int D>
__device__ __forceinline__ void dyadic5_msb(uint32_t M, uint32_t& e0, uint32_t& e1) {
  if constexpr (D == 0) {
    e0 = M << 4;
    e1 = M << 3;
  } else if constexpr (D == 1) {
    e0 = M << 2;
    e1 = M << 1;
  } else if constexpr (D == 2) {
    e0 = M >> 4;
    e1 = M >> 5;
  } else {
    e0 = M >> 6;
    e1 = M >> 7;
  }
}

// One packed dword + its high bits -> 8 bf16 values in SIGMA order (scales
// below 2^120).
__device__ __forceinline__ u32x4 dyadic5_rebuild_fma(uint32_t p, uint32_t e0, uint32_t e1,
                                                     const Dyadic5Scale& d) {
  const uint32_t q = p >> 8;
  const uint32_t mg = kMagic;
  u32x4 r;
  r.x = fma_pair(and_or(p, 0x000F000Fu, and_or(e0, 0x00100010u, mg)), d.s16, d.c1);
  r.y = fma_pair(and_or(p, 0x00F000F0u, and_or(e0, 0x01000100u, mg)), d.s256, d.c2);
  r.z = fma_pair(and_or(q, 0x000F000Fu, and_or(e1, 0x00100010u, mg)), d.s16, d.c1);
  r.w = fma_pair(and_or(q, 0x00F000F0u, and_or(e1, 0x01000100u, mg)), d.s256, d.c2);
  return r;
}

// The same for any scale: an exact fp16 subtraction, then one product and one
// RNE per value.
__device__ __forceinline__ u32x4 dyadic5_rebuild(uint32_t p, uint32_t e0, uint32_t e1,
                                                 const Dyadic5Scale& d, float pz) {
  const uint32_t q = p >> 8;
  const uint32_t mg = kMagic;
  const uint32_t o1 = 0x64106410u;  // fp16 1040 twice
  const uint32_t o2 = 0x65006500u;  // fp16 1280 twice
  u32x4 r;
  r.x = sub_mul_pair(and_or(p, 0x000F000Fu, and_or(e0, 0x00100010u, mg)), o1, d.s16, pz);
  r.y = sub_mul_pair(and_or(p, 0x00F000F0u, and_or(e0, 0x01000100u, mg)), o2, d.s256, pz);
  r.z = sub_mul_pair(and_or(q, 0x000F000Fu, and_or(e1, 0x00100010u, mg)), o1, d.s16, pz);
  r.w = sub_mul_pair(and_or(q, 0x00F000F0u, and_or(e1, 0x01000100u, mg)), o2, d.s256, pz);
  return r;
}

// ---------------------------------------------------------------- LUT16
// Per-group table T[j] = RNE_bf16(s * L_j), split into a low-byte plane and a
// high-byte plane of 4 dwords each.
struct Lut16Table {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Lut16Table lut16_table(uint32_t sbits, const u32x4& l0, const u32x4& l1) {
  const float s = bf16_bits_to_f32(sbits);
  uint32_t pairs[8];
  const uint32_t lw[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = bf16_bits_to_f32(lw[i] & 0xFFFFu) * s;  // exact in fp32
    const float b = __builtin_bit_cast(float, lw[i] & 0xFFFF0000u) * s;
    pairs[i] = cvt_pk_bf16(a, b);  // entries 2i, 2i+1
  }
  Lut16Table t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // entries 4i..4i+3 live in pairs[2i] (4i, 4i+1) and pairs[2i+1] (4i+2, 4i+3)
    t.lo[i] = perm(pairs[2 * i + 1], pairs[2 * i], 0x06040200u);
    t.hi[i] = perm(pairs[2 * i + 1], pairs[2 * i], 0x07050301u);
  }
  return t;
}

// One packed dword -> 8 bf16 values in SIGMA order.
__device__ __forceinline__ u32x4 lut16_rebuild(uint32_t p, const Lut16Table& t) {
  const uint32_t q = p & 0x0F0F0F0Fu;            // k0 k2 k4 k6
  const uint32_t r = (p >> 4) & 0x0F0F0F0Fu;     // k1 k3 k5 k7
  const uint32_t qx = q ^ 0x08080808u, rx = r ^ 0x08080808u;
  const uint32_t qm = merge_sel(p >> 1), rm = merge_sel(p >> 5);
  const uint32_t ql = lookup16(t.lo[0], t.lo[1], t.lo[2], t.lo[3], q, qx, qm);
  const uint32_t qh = lookup16(t.hi[0], t.hi[1], t.hi[2], t.hi[3], q, qx, qm);
  const uint32_t rl = lookup16(t.lo[0], t.lo[1], t.lo[2], t.lo[3], r, rx, rm);
  const uint32_t rh = lookup16(t.hi[0], t.hi[1], t.hi[2], t.hi[3], r, rx, rm);
  u32x4 o;
  o.x = perm(qh, ql, 0x06020400u);  // (k0, k4): lo byte q0, hi byte q0, lo q2, hi q2
  o.y = perm(rh, rl, 0x06020400u);  // (k1, k5)
  o.z = perm(qh, ql, 0x07030501u);  // (k2, k6)
  o.w = perm(rh, rl, 0x07030501u);  // (k3, k7)
  return o;
}

// ---------------------------------------------------------------- byte -> pair table
// LUT16S decoded a byte at a time: entry b of a 256-entry LDS table holds the
// two normalised levels (L[b & 15], L[b >> 4]) as fp32, so a packed byte
// yields its two weights with one LDS read, two products by the group scale
// (exact in fp32, as in lut16_table) and one conversion (the one RNE).  One
// packed dword -> 8 bf16 values in natural k order.
__device__ __forceinline__ u32x4 pair_rebuild(uint32_t p, float s, const f32x2* tab) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 v = tab[(p >> (8 * i)) & 0xFFu];
    r[i] = cvt_pk_bf16(v.x * s, v.y * s);
  }
  return r;
}

// ---------------------------------------------------------------- SIGNMAG8
// w_hat = +-M[mag] in fp16.  bf16 MFMA needs bf16 operands, so every fp16 level
// is split exactly as M = H + Lo with H = RNE_bf16(M) and Lo = M - H (at most 3
// significant bits, exact in bf16); the MFMA is issued on both halves and the
// fp32 accumulator receives x*H + x*Lo = x*M exactly per product.
// Tables: 8 entries -> 2 dwords per byte plane, for H and for Lo.
struct SignMagTable {
  uint32_t hl[2], hh[2], ll[2], lh[2];
};

__device__ __forceinline__ SignMagTable signmag_table(const u32x4& cb) {
  const uint32_t cw[4] = {cb.x, cb.y, cb.z, cb.w};
  uint32_t hp[4], lp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 m = __builtin_bit_cast(f16x2, cw[i]);
    const float a = (float)m.x, b = (float)m.y;
    hp[i] = cvt_pk_bf16(a, b);
    const float ha = bf16_bits_to_f32(hp[i] & 0xFFFFu);
    const float hb = __builtin_bit_cast(float, hp[i] & 0xFFFF0000u);
    lp[i] = cvt_pk_bf16(a - ha, b - hb);  // exact differences
  }
  SignMagTable t;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    t.hl[i] = perm(hp[2 * i + 1], hp[2 * i], 0x06040200u);
    t.hh[i] = perm(hp[2 * i + 1], hp[2 * i], 0x07050301u);
    t.ll[i] = perm(lp[2 * i + 1], lp[2 * i], 0x06040200u);
    t.lh[i] = perm(lp[2 * i + 1], lp[2 * i], 0x07050301u);
  }
  return t;
}

// One packed dword -> H and Lo operands (8 bf16 each, SIGMA order).
__device__ __forceinline__ void signmag_rebuild(uint32_t p, const SignMagTable& t, u32x4& H,
                                                u32x4& L) {
  const uint32_t q = p & 0x07070707u;          // magnitudes of k0 k2 k4 k6
  const uint32_t r = (p >> 4) & 0x07070707u;   // magnitudes of k1 k3 k5 k7
  const uint32_t qs = (p << 4) & 0x80808080u;  // sign bits of k0 k2 k4 k6 -> bit 7 of each byte
  const uint32_t rs = p & 0x80808080u;         // sign bits of k1 k3 k5 k7
  const uint32_t qhl = perm(t.hl[1], t.hl[0], q), qhh = perm(t.hh[1], t.hh[0], q) ^ qs;
  const uint32_t rhl = perm(t.hl[1], t.hl[0], r), rhh = perm(t.hh[1], t.hh[0], r) ^ rs;
  const uint32_t qll = perm(t.ll[1], t.ll[0], q), qlh = perm(t.lh[1], t.lh[0], q) ^ qs;
  const uint32_t rll = perm(t.ll[1], t.ll[0], r), rlh = perm(t.lh[1], t.lh[0], r) ^ rs;
  H.x = perm(qhh, qhl, 0x06020400u);
  H.y = perm(rhh, rhl, 0x06020400u);
  H.z = perm(qhh, qhl, 0x07030501u);
  H.w = perm(rhh, rhl, 0x07030501u);
  L.x = perm(qlh, qll, 0x06020400u);
  L.y = perm(rlh, rll, 0x06020400u);
  L.z = perm(qlh, qll, 0x07030501u);
  L.w = perm(rlh, rll, 0x07030501u);
}

// ---------------------------------------------------------------- activations
// 8 consecutive bf16 x values (natural order, 4 dwords) -> SIGMA order.
__device__ __forceinline__ u32x4 x_to_sigma(const u32x4& x) {
  u32x4 r;
  r.x = perm(x.z, x.x, 0x05040100u);  // (k0, k4)
  r.y = perm(x.z, x.x, 0x07060302u);  // (k1, k5)
  r.z = perm(x.w, x.y, 0x05040100u);  // (k2, k6)
  r.w = perm(x.w, x.y, 0x07060302u);  // (k3, k7)
  return r;
}

// SIGMA order -> natural order (for the dense dequant output).
__device__ __forceinline__ u32x4 sigma_to_natural(const u32x4& s) {
  u32x4 r;
  r.x = perm(s.y, s.x, 0x05040100u);  // (k0, k1) = lo(s.x), lo(s.y)
  r.y = perm(s.w, s.z, 0x05040100u);  // (k2, k3)
  r.z = perm(s.y, s.x, 0x07060302u);  // (k4, k5) = hi(s.x), hi(s.y)
  r.w = perm(s.w, s.z, 0x07060302u);  // (k6, k7)
  return r;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the wave wait for every vector-memory load in flight;
// here prefetched weight loads stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// D[32][32] += A[32][16] B[16][32].  A lane l: row l % 32, k = 8 (l / 32) .. +7;
// B lane l: column l % 32, the same k; D lane l register r: row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.  On gfx950 this shape retires
// twice the bf16 flops per cycle of the 16x16x32 one.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace w4
