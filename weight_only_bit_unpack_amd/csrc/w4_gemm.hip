// Fused dequant + GEMM for prefill-sized batches (gfx950).
//
// k-means page, section 4.1: batches above the LUT-kernel range go to a mixed
// 4-bit x bf16 kernel.  Y[M][N] = X[M][K] * W_hat[N][K]^T, bf16 MFMA with fp32
// accumulation; each 4-bit weight is rebuilt (w4_device.h) once per block into
// LDS and multiplied there against every batch row of the block.
//
// Block tile 256 (batch rows) x 128 (weight rows), k-step 64 (one 64-group per
// weight row), one block per CU with eight waves, two per SIMD.  Wave w owns
// batch rows 64 (w % 4) .. + 63 against all 128 weight rows = 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane), for half of each
// k-step (w / 4); the two halves are added through LDS after the k loop.  Two
// waves per SIMD let one wave's MFMAs run while the other waits on memory,
// LDS or the rebuild, which a single wave cannot overlap.  Batches of at most
// 128 rows use a 128 x 128 block with 128-k steps instead: four waves share a
// row group, one k quarter each, so every wave's work per step is the same.
//
// A wave owns its batch rows, so its activation operands come straight from
// global memory into registers, from a copy of x rewritten once per call into
// MFMA operand order (pack_activations); only the rebuilt weights go through
// LDS: 16 KB of writes and 64 KB of reads per k-step against 4.2 MFLOP of MFMA
// work.  Within every 8 consecutive k both operands hold their values in the
// rebuild's slot order SIGMA (w4_device.h): the contraction only needs the two
// sides to agree on the k order, and the weights are then stored as rebuilt.
//
// The k range is split over S blocks when the output tiles alone cannot fill
// the GPU (256 x 8192 outputs are only 64 tiles); each split writes an fp32
// partial in the MFMA register layout and a second kernel adds the partials in
// split order, so results do not depend on timing.
//
// Software pipeline: weights are loaded four k-steps ahead and activations
// one step ahead; the rebuilt weights are double-buffered in LDS, and each
// step's block barrier sits between its two 16-k halves of MFMAs, so that the
// LDS reads of the next step's operands run under the current step's MFMAs
// (details at the loop).  Loads past the block's k range use offsets past the
// buffer resource and return zero, so the loop runs whole rounds of four steps
// without branches.
#include "w4_device.h"
#include "w4_launch.h"

#include <atomic>
#include <type_traits>


namespace w4 {
namespace {

constexpr int BN = 128;  // weight rows per block
constexpr int kMaxSplits = 8;
constexpr uint32_t kOOB = 0x80000000u;

// Block shapes by batch rows per block.  BMT = 256: four row groups of 64
// batch rows, each shared by two waves that take the two k halves of a 64-k
// step.  BMT = 128: two row groups, each shared by four waves that take the
// four k quarters of a 128-k step.  Either way a wave computes 64 x 128
// outputs over 32 k per step (16 MFMAs), and each thread rebuilds BK / 4
// weights of one weight row per step.
template <int BMT>
struct Tile {
  static constexpr int MW = BMT / 64;     // row groups
  static constexpr int KW = 8 / MW;       // waves (k parts) per row group
  static constexpr int BK = 32 * KW;      // k per step
  static constexpr int DW = BK / 32;      // packed dwords a thread rebuilds per step
  static constexpr int STR = BK / 8 + 1;  // 16-byte units per LDS weight row (+1: conflict-free reads)
  static constexpr int WS = BN * STR;     // 16-byte units per weight tile plane
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Per-thread constants of the rebuild: the one 16-level table of a LUT16S
// weight; for DYADIC5, the shift that brings the thread's half of a run's
// high-bit word to the position its first packed dword expects.
struct RebuildConsts {
  u32x4 l0, l1;
  uint32_t msb_shift;
};

// Packed bytes and side data one thread rebuilds per k-step: weight row
// tid / 4, k = 8 DW (tid % 4) .. + 8 DW - 1 of the step (DW packed dwords, all
// in one 64-group and one 32-group run).  The rebuilt values go to LDS in
// SIGMA order, as the activations are packed.
template <int CODEC, int DW>
struct WRaw;

template <int DW>
__device__ __forceinline__ void load_packed(uint32_t (&p)[DW], __amdgpu_buffer_rsrc_t pk,
                                            uint32_t po) {
  static_assert(DW == 2 || DW == 4, "two or four packed dwords");
  if constexpr (DW == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(pk, po, 0, 0);
    p[0] = v[0];
    p[1] = v[1];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(pk, po, 0, 0);
    p[0] = v[0];
    p[1] = v[1];
    p[2] = v[2];
    p[3] = v[3];
  }
}

template <int DW>
struct WRaw<0, DW> {  // DYADIC: bf16 scale of the row's 64-group
  uint32_t p[DW];
  uint16_t sb;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t pk, __amdgpu_buffer_rsrc_t s0,
                                       __amdgpu_buffer_rsrc_t, uint32_t po, uint32_t so,
                                       uint32_t) {
    load_packed<DW>(p, pk, po);
    sb = __builtin_amdgcn_raw_buffer_load_b16(s0, so, 0, 0);
  }
  template <int D>
  __device__ __forceinline__ void rebuild(u32x4& hi, u32x4&, const RebuildConsts&) const {
    const DyadicScale d = dyadic_scale(sb);
    const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, mg = kMagic;
    const float nz = __builtin_bit_cast(float, opaque(0x80000000u));
    hi = dyadic_rebuild_any(p[D], d, m0, m1, mg, nz);
  }
};

template <int DW>
struct WRaw<1, DW> {  // LUT16: 16 bf16 levels + bf16 scale of the row's 64-group
  uint32_t p[DW];
  u32x4 l0, l1;
  uint16_t sb;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t pk, __amdgpu_buffer_rsrc_t s0,
                                       __amdgpu_buffer_rsrc_t s1, uint32_t po, uint32_t so,
                                       uint32_t co) {
    load_packed<DW>(p, pk, po);
    l0 = __builtin_amdgcn_raw_buffer_load_b128(s1, co, 0, 0);
    l1 = __builtin_amdgcn_raw_buffer_load_b128(s1, co + 16, 0, 0);
    sb = __builtin_amdgcn_raw_buffer_load_b16(s0, so, 0, 0);
  }
  template <int D>
  __device__ __forceinline__ void rebuild(u32x4& hi, u32x4&, const RebuildConsts&) const {
    const Lut16Table t = lut16_table(sb, l0, l1);
    hi = lut16_rebuild(p[D], t);
  }
};

template <int DW>
struct WRaw<2, DW> {  // SIGNMAG8: 8 fp16 magnitudes of the row's 32-group
  uint32_t p[DW];
  u32x4 c;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t pk, __amdgpu_buffer_rsrc_t,
                                       __amdgpu_buffer_rsrc_t s1, uint32_t po, uint32_t,
                                       uint32_t co) {
    load_packed<DW>(p, pk, po);
    c = __builtin_amdgcn_raw_buffer_load_b128(s1, co, 0, 0);
  }
  template <int D>
  __device__ __forceinline__ void rebuild(u32x4& hi, u32x4& lo, const RebuildConsts&) const {
    const SignMagTable t = signmag_table(c);
    signmag_rebuild(p[D], t, hi, lo);
  }
};

template <int DW>
struct WRaw<3, DW> {  // LUT16S: bf16 scale of the row's 64-group; levels shared
  uint32_t p[DW];
  uint16_t sb;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t pk, __amdgpu_buffer_rsrc_t s0,
                                       __amdgpu_buffer_rsrc_t, uint32_t po, uint32_t so,
                                       uint32_t) {
    load_packed<DW>(p, pk, po);
    sb = __builtin_amdgcn_raw_buffer_load_b16(s0, so, 0, 0);
  }
  template <int D>
  __device__ __forceinline__ void rebuild(u32x4& hi, u32x4&, const RebuildConsts& st) const {
    const Lut16Table t = lut16_table(sb, st.l0, st.l1);
    hi = lut16_rebuild(p[D], t);
  }
};

template <int DW>
struct WRaw<4, DW> {  // DYADIC5: bf16 scale of the row's 64-group + high-bit word of its run of 32
  uint32_t p[DW], h;
  uint16_t sb;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t pk, __amdgpu_buffer_rsrc_t s0,
                                       __amdgpu_buffer_rsrc_t s1, uint32_t po, uint32_t so,
                                       uint32_t co) {
    load_packed<DW>(p, pk, po);
    sb = __builtin_amdgcn_raw_buffer_load_b16(s0, so, 0, 0);
    h = __builtin_amdgcn_raw_buffer_load_b32(s1, co, 0, 0);
  }
  // DW = 2: dword D of the thread's 16 weights is dword 2 (wq % 2) + D of the
  // run, and msb_shift (0 or 8) folds the 2 (wq % 2) into the shifts of dwords
  // 0, 1.  DW = 4: the thread's dwords are the whole run, msb_shift 0.
  template <int D>
  __device__ __forceinline__ void rebuild(u32x4& hi, u32x4&, const RebuildConsts& c) const {
    uint32_t e0, e1;
    dyadic5_msb<D>(h >> c.msb_shift, e0, e1);
    const float pz = __builtin_bit_cast(float, opaque(0u));
    hi = dyadic5_rebuild(p[D], e0, e1, dyadic5_scale(sb), pz);
  }
};

// LDS: two rebuilt weight tiles during the k loop; after it, the same bytes
// hold the k-part partial sums that the waves of one row group exchange (one
// 32 KB slot per writing wave: four row groups x one for BMT = 256, two row
// groups x two for BMT = 128).
constexpr size_t kRedSlotBytes = 32 * 64 * 16;  // 128 floats x 64 lanes
template <int CODEC, int BMT>
constexpr size_t gemm_lds_bytes() {
  const size_t w = (size_t)2 * (CODEC == 2 ? 2 : 1) * Tile<BMT>::WS * 16;
  const size_t r = (size_t)4 * kRedSlotBytes;
  return w > r ? w : r;
}

template <int D>
using DI = std::integral_constant<int, D>;

template <int CODEC, int BMT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(
    GemvProblem P, int M, int y_bf16, const u32x4* __restrict__ xpk, float* __restrict__ partial) {
  using TL = Tile<BMT>;
  constexpr int MW = TL::MW, KW = TL::KW, BK = TL::BK, DW = TL::DW, STR = TL::STR;
  constexpr int NPL = CODEC == 2 ? 2 : 1;  // SIGNMAG8: high and low bf16 planes
  extern __shared__ u32x4 lds[];
  auto wtile = [&](int buf, int pl) { return lds + (buf * NPL + pl) * TL::WS; };

  const int64_t N = P.n, K = P.k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mw = wave % MW, kh = wave / MW;  // row group, k part
  // Block -> (split, n tile, m tile), m fastest.  Blocks are dealt to the 8
  // XCDs round robin; renumbering them so that each XCD gets a contiguous
  // range of this order keeps one split's activations (BMT x k / S bf16 per m
  // tile) in that XCD's L2 instead of all of them, and the m tiles of one
  // weight tile on the same XCD, which then reads those weights from HBM once.
  const uint32_t G = gridDim.x, b = blockIdx.x;
  const uint32_t L = (G & 7u) == 0 ? (b & 7u) * (G >> 3) + (b >> 3) : b;
  const uint32_t tiles_n = (uint32_t)((P.n + BN - 1) / BN), tiles_m = (uint32_t)((M + BMT - 1) / BMT);
  const uint32_t tile = L % (tiles_n * tiles_m);
  const uint32_t nt = tile / tiles_m, mt = tile % tiles_m;
  const int s = (int)(L / (tiles_n * tiles_m));
  const int64_t n0 = (int64_t)nt * BN, m0 = (int64_t)mt * BMT;
  const int rows_n = (int)(N - n0 < BN ? N - n0 : BN);
  const int rows_m = (int)(M - m0 < BMT ? M - m0 : BMT);

  // k range of this split, in BK steps (k is a multiple of BK)
  const int T = (int)(K / BK), S = (int)(G / (tiles_n * tiles_m));
  const int ks0 = (int)((int64_t)s * T / S), ks1 = (int)((int64_t)(s + 1) * T / S);
  const int nsteps = ks1 - ks0;

  // weight rebuild role: row wr, part wq (DW packed dwords) of the step
  const int wr = tid >> 2, wq = tid & 3;
  const uint32_t row_bytes = (uint32_t)(K >> 1);
  const __amdgpu_buffer_rsrc_t pk = rsrc(P.packed + n0 * (K >> 1), (uint32_t)rows_n * row_bytes);
  __amdgpu_buffer_rsrc_t s0 = pk, s1 = pk;
  if constexpr (CODEC == 0 || CODEC == 3) {
    s0 = rsrc(P.scales + n0 * (K >> 6), (uint32_t)(rows_n * (K >> 6) * 2));
  } else if constexpr (CODEC == 4) {
    s0 = rsrc(P.scales + n0 * (K >> 6), (uint32_t)(rows_n * (K >> 6) * 2));
    s1 = rsrc(reinterpret_cast<const uint8_t*>(P.codebook) + n0 * (K >> 3),
              (uint32_t)(rows_n * (K >> 3)));
  } else if constexpr (CODEC == 1) {
    s0 = rsrc(P.scales + n0 * (K >> 6), (uint32_t)(rows_n * (K >> 6) * 2));
    s1 = rsrc(P.codebook + n0 * (K >> 6) * 16, (uint32_t)(rows_n * (K >> 6) * 32));
  } else {
    s1 = rsrc(P.codebook + n0 * (K >> 5) * 8, (uint32_t)(rows_n * (K >> 5) * 16));
  }
  // the thread's bytes of a step and their 64-group and run of 32; per step
  // these advance by BK / 2 bytes, BK / 64 groups and BK / 32 runs
  constexpr uint32_t kPkStep = BK / 2, kG64Step = BK / 64, kG32Step = BK / 32;
  const uint32_t p_lane = (uint32_t)wr * row_bytes + 4u * DW * (uint32_t)wq;
  const uint32_t g64_lane = (uint32_t)wr * (uint32_t)(K >> 6) + (uint32_t)(wq * DW / 8);
  const uint32_t g32_lane = (uint32_t)wr * (uint32_t)(K >> 5) + (uint32_t)(wq * DW / 4);
  // DYADIC5: byte offset of the high-bit word of the thread's run of 32
  const uint32_t h_lane = (uint32_t)wr * (uint32_t)(K >> 3) + 4u * (uint32_t)(wq * DW / 4);

  // activation role: the block's BMT / 32 row tiles of 32 in the packed layout
  // (pack_activations); wave (mw, kh) takes row tiles 2 mw + i and, within a
  // step, 16-k blocks kb = 2 kh + kk
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t kblocks = (uint32_t)(K >> 4);
  const __amdgpu_buffer_rsrc_t xr =
      rsrc(xpk + (size_t)(m0 >> 5) * kblocks * 64, (uint32_t)(BMT / 32) * kblocks * 1024u);
  const uint32_t x_lane = ((uint32_t)(2 * mw) * kblocks + 2u * (uint32_t)kh) * 1024u + 16u * (uint32_t)lane;
  const uint32_t x_i = kblocks * 1024u;  // next row tile
  constexpr uint32_t kXStep = 64u * BK;  // BK / 16 records of 1 KB per step

  WRaw<CODEC, DW> wqr[4];
  u32x4 xq[2][2][2];
  // Offsets of a step past the split are kOOB plus at most 2^31 - 1: still
  // past every resource (num_records <= 2^31 since k <= 2^22), so those loads
  // return zero without a branch.
  auto load_w = [&](WRaw<CODEC, DW>& r, int u) {
    const bool in = u < nsteps;
    const uint32_t ks = (uint32_t)(ks0 + u);
    // byte offsets: packed, 64-group scale, codebook (LUT16 levels / SIGNMAG8 magnitudes)
    const uint32_t co = CODEC == 1   ? 32u * (g64_lane + kG64Step * ks)
                        : CODEC == 4 ? h_lane + 4u * kG32Step * ks
                                     : 16u * (g32_lane + kG32Step * ks);
    r.load(pk, s0, s1, opaque(in ? p_lane + ks * kPkStep : kOOB),
           opaque(in ? 2u * (g64_lane + kG64Step * ks) : kOOB), opaque(in ? co : kOOB));
  };
  auto load_x = [&](u32x4 (&xv)[2][2], int u) {
    const bool in = u < nsteps;
    const uint32_t base = opaque(in ? x_lane + (uint32_t)(ks0 + u) * kXStep : kOOB);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        xv[i][kk] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, base + (uint32_t)i * x_i + (uint32_t)kk * 1024u, 0, 0);
  };
  RebuildConsts st{};
  st.msb_shift = DW == 2 ? 8u * (uint32_t)(wq & 1) : 0u;
  if constexpr (CODEC == 3) {
    st.l0 = reinterpret_cast<const u32x4*>(P.codebook)[0];
    st.l1 = reinterpret_cast<const u32x4*>(P.codebook)[1];
  }
  // rebuild packed dword D (k = 8 (DW wq + D) .. + 7 of the step) into LDS
  auto rebuild = [&](const WRaw<CODEC, DW>& r, int buf, auto dtag) {
    constexpr int D = decltype(dtag)::value;
    u32x4 hi, lo;
    r.template rebuild<D>(hi, lo, st);
    wtile(buf, 0)[wr * STR + DW * wq + D] = hi;
    if constexpr (NPL == 2) wtile(buf, 1)[wr * STR + DW * wq + D] = lo;
  };
  // the first and the second half of a thread's dwords
  auto rebuild_first = [&](const WRaw<CODEC, DW>& r, int buf) {
    rebuild(r, buf, DI<0>{});
    if constexpr (DW == 4) rebuild(r, buf, DI<1>{});
  };
  auto rebuild_second = [&](const WRaw<CODEC, DW>& r, int buf) {
    if constexpr (DW == 2) {
      rebuild(r, buf, DI<1>{});
    } else {
      rebuild(r, buf, DI<2>{});
      rebuild(r, buf, DI<3>{});
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // B operands of one 16-k block kk of the wave's k part (4 weight-row tiles of 32)
  auto read_b = [&](u32x4 (&bq)[NPL][4], int buf, int kk) {
    const int kb = 2 * kh + kk;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[pl][j] = wtile(buf, pl)[(32 * j + r32) * STR + 2 * kb + h];
  };
  auto mma_half = [&](const u32x4 (&xv)[2][2], const u32x4 (&bq)[NPL][4], int kk) {
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(xv[i][kk], bq[pl][j], acc[i][j]);
  };

  // Each k-step u runs in two phases split by the block barrier:
  //   A(u): reads of B(u, second 16-k block); MFMAs of the first block; the
  //         second half of step u+1's rebuild (so all of u+1 is in LDS at the
  //         barrier); the loads of step u+4 (weights) and u+1 (activations).
  //   B(u): reads of B(u+1, first block), right after the barrier; MFMAs of
  //         u's second block; the first half of step u+2's rebuild into the
  //         buffer step u has just released.
  // The LDS reads of the next step thus run under the MFMAs of the current
  // one instead of between barriers, and each phase's rebuild work (about
  // half a step's VALU) runs beside its eight MFMAs per wave.
  u32x4 b0[NPL][4], b1[NPL][4];
  load_w(wqr[0], 0);
  load_w(wqr[1], 1);
  load_w(wqr[2], 2);
  load_w(wqr[3], 3);
  load_x(xq[0], 0);
  rebuild_first(wqr[0], 0);
  rebuild_second(wqr[0], 0);
  rebuild_first(wqr[1], 1);
  lds_barrier();
  read_b(b0, 0, 0);

  for (int u = 0; u < nsteps; u += 4) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int cur = v & 1, nxt = (v + 1) & 1;
      // phase A
      read_b(b1, cur, 1);
      load_x(xq[nxt], u + v + 1);
      mma_half(xq[cur], b0, 0);
      rebuild_second(wqr[(v + 1) & 3], nxt);
      load_w(wqr[v & 3], u + v + 4);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // phase B
      read_b(b0, nxt, 0);
      mma_half(xq[cur], b1, 1);
      rebuild_first(wqr[(v + 2) & 3], cur);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();  // the last phase's LDS traffic is done before LDS is reused

  // the k parts of a row group meet in LDS (the weight tiles are dead):
  // BMT = 256 adds a0 + a1; BMT = 128 adds (a0 + a1) + (a2 + a3)
  auto put = [&](int slot) {
    f32x4* const d = reinterpret_cast<f32x4*>(lds) + slot * 32 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& a = acc[i][j];
          d[((i * 4 + j) * 4 + r4) * 64] =
              (f32x4){a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
        }
  };
  auto add = [&](int slot) {
    const f32x4* const d = reinterpret_cast<const f32x4*>(lds) + slot * 32 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 o = d[((i * 4 + j) * 4 + r4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * r4 + e] += o[e];
        }
  };
  if constexpr (KW == 2) {
    if (kh == 1) put(mw);
    lds_barrier();
    if (kh == 1) return;
    add(mw);
  } else {
    if (kh & 1) put(2 * mw + (kh >> 1));
    lds_barrier();
    if (!(kh & 1)) add(2 * mw + (kh >> 1));
    lds_barrier();
    if (kh == 2) put(mw);  // slots 0, 1: read in the first round already
    lds_barrier();
    if (kh != 0) return;
    add(mw);
  }

  if (partial) {
    // split partial in the MFMA register layout: 16-byte stores, 1 KB per
    // instruction; the reduction kernel maps it back to rows and columns
    f32x4* dst = reinterpret_cast<f32x4*>(partial) +
                 (((size_t)s * tiles_m * tiles_n + tile) * MW + mw) * 32 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& a = acc[i][j];
          dst[((i * 4 + j) * 4 + r4) * 64] =
              (f32x4){a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
        }
    return;
  }
  // D[m][n] of tile (i, j) sits in lane n + 32 ((m / 4) % 2), register
  // 4 (m / 8) + m % 4
  float* const yf = reinterpret_cast<float*>(P.y);
  uint16_t* const yh = reinterpret_cast<uint16_t*>(P.y);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cn = 32 * j + r32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rm = 64 * mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (cn < rows_n && rm < rows_m) {
          const int64_t o = (m0 + rm) * N + n0 + cn;
          if (y_bf16)
            yh[o] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
          else
            yf[o] = acc[i][j][r];
        }
      }
  }
}

// Activations in MFMA operand order: for each 32-row tile R and 16-k block B
// a 1 KB record whose lane l holds x[32 R + l % 32][16 B + 8 (l / 32) .. + 7]
// in SIGMA order (rows past M are zero).  The GEMM then reads every operand as 1 KB of
// contiguous memory; read straight from x, each operand load would touch 32
// rows and the L1 would stall the address path.
__global__ __launch_bounds__(256) void pack_activations(const u32x4* __restrict__ x,
                                                        u32x4* __restrict__ xpk, int64_t M,
                                                        int64_t K) {
  // block = (row tile R, 64-k slab c): 32 rows x 128 bytes read row-contiguous
  // into LDS, written out as the slab's four 1 KB records
  __shared__ u32x4 t[32][9];
  const int tid = threadIdx.x;
  const int64_t kblocks = K >> 4, slabs = K >> 6;
  const int64_t R = (int64_t)blockIdx.x / slabs, c = (int64_t)blockIdx.x % slabs;
  {
    const int r = tid >> 3, u = tid & 7;
    const int64_t row = R * 32 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < M) v = x[(row * K + c * 64) / 8 + u];
    t[r][u] = v;
  }
  __syncthreads();
  const int rec = tid >> 6, lane = tid & 63;  // record rec = 16-k block 4c + rec
  xpk[(R * kblocks + 4 * c + rec) * 64 + lane] = x_to_sigma(t[lane & 31][2 * rec + (lane >> 5)]);
}

// y = sum of the S split partials, added in split order.  One thread per
// (tile, row group, 4-register group, lane) of the GEMM's register layout.
template <int BMT>
__global__ __launch_bounds__(256) void splitk_reduce(const f32x4* __restrict__ partial, int S,
                                                     uint32_t tiles_m, uint32_t tiles,
                                                     int64_t M, int64_t N, void* y, int y_bf16) {
  constexpr int MW = Tile<BMT>::MW;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // < tiles * MW * 32 * 64
  const int64_t per_split = (int64_t)tiles * MW * 32 * 64;
  if (t >= per_split) return;
  // every split's load in flight at once, then the sum in split order
  f32x4 p[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    p[s] = s < S ? partial[(int64_t)s * per_split + t] : (f32x4){0.f, 0.f, 0.f, 0.f};
  f32x4 v = p[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) v += p[s];
  const int lane = (int)(t & 63), r4g = (int)((t >> 6) & 31);
  const int mw = (int)((t >> 11) % MW);
  const uint32_t tile = (uint32_t)((t >> 11) / MW);
  const int r32 = lane & 31, h = lane >> 5;
  const int i = r4g >> 4, j = (r4g >> 2) & 3, r4 = r4g & 3;
  const int64_t row0 = (int64_t)(tile % tiles_m) * BMT + 64 * mw + 32 * i + 8 * r4 + 4 * h;
  const int64_t col = (int64_t)(tile / tiles_m) * BN + 32 * j + r32;
  if (col >= N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t row = row0 + e;
    if (row < M) {
      if (y_bf16)
        reinterpret_cast<uint16_t*>(y)[row * N + col] = (uint16_t)f32_to_bf16_bits(v[e]);
      else
        reinterpret_cast<float*>(y)[row * N + col] = v[e];
    }
  }
}

// Splits of the k range: enough blocks for about one per CU, at least eight
// k-steps per split, at most eight splits.
int gemm_splits(int64_t n, int64_t k, int m, int cus, int bm, int bk) {
  const int64_t tiles = ((n + BN - 1) / BN) * ((m + bm - 1) / bm);
  const int64_t steps = k / bk;
  int64_t s = tiles > 0 ? (cus + tiles - 1) / tiles : 1;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > steps / 8) s = steps / 8;
  return s < 1 ? 1 : (int)s;
}

template <int CODEC, int BMT>
hipError_t launch_codec(const GemvProblem& p, int m, int y_bf16, const u32x4* xpk, float* partial,
                        uint32_t blocks, hipStream_t stream) {
  constexpr size_t lds = gemm_lds_bytes<CODEC, BMT>();
  // the LDS limit is raised once per device (one bit each for the first 64);
  // callers racing here all set the same value
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t{1} << dev : 0;
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<CODEC, BMT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_release);
  }
  gemm_kernel<CODEC, BMT><<<dim3(blocks), dim3(512), lds, stream>>>(p, m, y_bf16, xpk, partial);
  return hipGetLastError();
}

// The 128-row block serves batches of at most 128 rows, which would leave half
// of a 256-row block's MFMA work on zero rows, for the codecs whose side data
// fits the registers of its four packed dwords per thread (all but SIGNMAG8,
// whose two operand planes leave none) when k is a multiple of its 128-k step.  Measured at K = N = 8192:
// M = 128 in 34 us against 45 us; at M = 256 its halved k splits do not make
// up for the doubled rebuild work per step (about 3% slower), and it is
// slower still at M = 512 and 1024.
constexpr int kNarrowMaxM = 128;
bool gemm_narrow(int codec, int64_t k, int m) {
  return (codec == 0 || codec == 1 || codec == 3 || codec == 4) && k % 128 == 0 && m <= kNarrowMaxM;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return cus;
}

// Workspace of one call: packed activations of tiles_m * BMT rows, then S
// fp32 partials of tiles * BMT * BN when the k range is split.
template <int BMT>
struct GemmPlan {
  int S;
  uint32_t tiles_m, tiles_n, tiles;
  size_t xpk_bytes, per_split, bytes;
  GemmPlan(int64_t n, int64_t k, int m, int cus) {
    S = gemm_splits(n, k, m, cus, BMT, Tile<BMT>::BK);
    tiles_n = (uint32_t)((n + BN - 1) / BN);
    tiles_m = (uint32_t)((m + BMT - 1) / BMT);
    tiles = tiles_n * tiles_m;
    xpk_bytes = (size_t)tiles_m * BMT * k * 2;
    per_split = (size_t)tiles * BMT * BN;  // floats
    bytes = xpk_bytes + (S > 1 ? (size_t)S * per_split * sizeof(float) : 0);
  }
};

// ws: the caller's workspace of at least GemmPlan::bytes, or nullptr for the
// stream's library-kept one
template <int BMT>
hipError_t launch_gemm_shape(int codec, const GemvProblem& p, int m, int y_bf16,
                             hipStream_t stream, char* ws) {
  const GemmPlan<BMT> g(p.n, p.k, m, device_cus());
  const int S = g.S;
  const uint32_t tiles_m = g.tiles_m, tiles = g.tiles;
  const size_t xpk_bytes = g.xpk_bytes, per_split = g.per_split;
  hipError_t e = hipSuccess;
  if (!ws) {
    e = stream_workspace(kWorkspaceGemm, stream, g.bytes, &ws);
    if (e != hipSuccess) return e;
  }
  u32x4* xpk = reinterpret_cast<u32x4*>(ws);
  float* partial = S > 1 ? reinterpret_cast<float*>(ws + xpk_bytes) : nullptr;
  pack_activations<<<dim3((uint32_t)(tiles_m * (BMT / 32) * (p.k / 64))), dim3(256), 0, stream>>>(
      reinterpret_cast<const u32x4*>(p.x), xpk, m, p.k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t blocks = tiles * (uint32_t)S;
  if (codec == 0)
    e = launch_codec<0, BMT>(p, m, y_bf16, xpk, partial, blocks, stream);
  else if (codec == 3)
    e = launch_codec<3, BMT>(p, m, y_bf16, xpk, partial, blocks, stream);
  else if (codec == 4)
    e = launch_codec<4, BMT>(p, m, y_bf16, xpk, partial, blocks, stream);
  else if (codec == 1)
    e = launch_codec<1, BMT>(p, m, y_bf16, xpk, partial, blocks, stream);
  else if constexpr (BMT == 256) {
    e = launch_codec<2, 256>(p, m, y_bf16, xpk, partial, blocks, stream);
  } else {
    return hipErrorInvalidValue;  // SIGNMAG8 uses the 256-row block only
  }
  if (e != hipSuccess || S == 1) return e;
  const size_t threads = per_split / 4;
  splitk_reduce<BMT><<<dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, stream>>>(
      reinterpret_cast<const f32x4*>(partial), S, tiles_m, tiles, m, p.n, p.y, y_bf16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream,
                       char* ws) {
  if (gemm_narrow(codec, p.k, m)) return launch_gemm_shape<128>(codec, p, m, y_bf16, stream, ws);
  return launch_gemm_shape<256>(codec, p, m, y_bf16, stream, ws);
}

size_t gemm_workspace_bytes(int codec, int64_t n, int64_t k, int m) {
  if (gemm_narrow(codec, k, m)) return GemmPlan<128>(n, k, m, device_cus()).bytes;
  return GemmPlan<256>(n, k, m, device_cus()).bytes;
}

}  // namespace w4
