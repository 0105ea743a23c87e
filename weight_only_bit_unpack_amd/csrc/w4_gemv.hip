// Fused dequant + GEMV for m <= 16 (gfx950).
//
// k-means page, section 4.1: a batch of m <= 16 goes to a dedicated 4-bit
// kernel; section 2.2: the weights are decoded on the fly from a small table.
// DyadicGumbel page, section 2.2: w = step * (idx - 8) per group of 64.
// int4-g32 page, section 5.2: a fused int4 kernel with the group codebook in
// registers.
//
// Work unit: a 16-row x 256-k step of one wave.  The wave loads its rows'
// packed bytes as whole 128-byte lines (Shuffle below) and moves them through
// LDS into MFMA lane order: lane l = (r = l % 16, q = l / 16) then holds the
// 32 packed bytes of row r covering k = 256 s + 64 q .. + 63 (one 64-group, or
// two 32-groups for SIGNMAG8).  Each of the lane's 8 packed dwords is rebuilt
// into one bf16 MFMA B operand (8 values), and v_mfma_f32_16x16x32_bf16
// multiplies it by the activation operand: A row = batch row m (rows >= m
// repeat row m-1 and are never stored), D[m][r] lands in lane r + 16 (m / 4),
// register m % 4.  For m = 1 the matrix core does 16x the necessary
// multiplies, which costs nothing here: the kernel is bound by HBM and by the
// VALU work of the rebuild (about 17 VALU instructions per 8 weights), and the
// MFMA takes the multiply-adds off the VALU.
//
// The activations are staged once per block into LDS in the rebuild's slot
// order (w4_device.h, SIGMA), in k-chunks when m * k does not fit.
// A block is max(4, KSPLIT) waves = KSPLIT waves along k x (waves / KSPLIT)
// row tiles of 16.  With KSPLIT > 1 the waves' partial sums are added in LDS
// in a fixed order.  KSPLIT = 4, 8 and 16 (one row tile per block of 4, 8 or
// 16 waves) serve single calls on matrices too short to fill the GPU with
// 64-row blocks (for m >= 2 when the activations fit the block's LDS): the
// waves of one 16-row tile take every 4th, 8th or 16th step.
#include "w4_device.h"
#include "w4_launch.h"


namespace w4 {
namespace {

// Staged activations: at most 3584 16-byte units (56 KiB) for a 4-wave block,
// so that with its four 2 KiB shuffle areas it stays within 64 KiB of LDS and
// two blocks share a CU; blocks of more waves keep the same 64 KiB total.
constexpr int kLdsBlockUnits = 4096;  // 64 KiB
constexpr int kXsUnitsMax = kLdsBlockUnits - 128 * 4;

// Buffer resources (V#) over one block's slice of an array: loads at an
// offset outside [0, num_records) return zero without touching memory, so
// rows past n and k past the end need no branches, and the compiler can
// keep prefetched loads in flight across the loop (vmcnt stays exact).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every slice
// Per-lane base offset of a load that must read zeros: kOOBLane plus any step
// offset (below 2^31, or kOOB itself) stays past every slice (slices hold
// fewer than 2^28 bytes) and below 2^32.
constexpr uint32_t kOOBLane = 0x40000000u;
// Cache policy of the packed-weight loads: nontemporal.  Every packed byte is
// read once per launch; streaming it leaves the caches to the scales and
// tables, which neighbouring lanes and steps read again (measured on the 1B
// decode stack: 3-4% faster; the same policy on the scale loads is slower).
constexpr int kPackedPolicy = 2;

// Offsets pass through an empty asm so the compiler keeps the select as one
// v_cndmask instead of splitting the loads into branches (which would make it
// wait for every outstanding load at the join).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Per-block view of one problem: resources rebased at the block's first row.
struct Slice {
  __amdgpu_buffer_rsrc_t packed, side, side2, x;
};

// Per-lane byte offsets of the lane's first step in the current k-chunk.
// Rows past the slice give offsets past num_records (reads return zero).
// When the block's k range does not end on a 256-k step (RAGGED kernels), the
// lanes of its last step whose weights lie past the range get base kOOBLane
// and read zeros: weights rebuilt from zero bytes and zero side data are
// finite, and meet zero activations in LDS.  (Read as they lie in memory,
// they would be the next row's weights, which may rebuild to +-inf.)
struct LaneBase {
  uint32_t pa, pb, s, s2;
};

// The packed bytes of a wave's 16 rows are loaded with whole 128-byte lines
// per row (8 lanes x 16 bytes, rows 0-7 then rows 8-15), which streams HBM far
// better than giving each MFMA lane its own 32 bytes straight from memory, and
// then moved into MFMA lane order (lane = row + 16 g holds bytes 32g..32g+31 of
// its row) through a 2 KiB per-wave LDS area.  Inside a row the 16-byte chunks
// are stored XOR-swizzled by (row >> 1) & 7 so the reads are bank-conflict free.
struct Shuffle {
  u32x4* stage;  // this wave's 128 x 16-byte area
  int wr, rd0, rd1;
  __device__ __forceinline__ void operator()(const u32x4& a0, const u32x4& a1, u32x4& p0,
                                             u32x4& p1) const {
    stage[wr] = a0;
    stage[64 + wr] = a1;
    p0 = stage[rd0];
    p1 = stage[rd1];
  }
};

// The one 16-level table of a LUT16S weight: as 16 bf16 levels in registers
// for the v_perm decode (LUT16S_PERM), as the block's 256-entry pair table in
// LDS for the byte -> pair decode (LUT16S, LUT16S_IL).
struct SharedTable {
  u32x4 l0, l1;
  const f32x2* tab;
};

// LUT16S weights are decoded a packed byte at a time through a 256-entry LDS
// table of level pairs (measured faster on the decode stack than the
// per-group byte-plane v_perm lookups of LUT16, which W4_LUT16S_PERM = 5
// keeps for comparison).  W4_LUT16S_IL = 6 is LUT16S with each row's scales
// interleaved into its packed bytes: per 256-k block a 144-byte record of 128
// bytes of nibbles, the block's four bf16 scales and 8 zero bytes.
constexpr uint32_t kIlRecord = 144;

// Raw per-step loads of one lane: 32 packed bytes plus the side data of the
// group(s) they belong to.  `sp` / `ss` are the step's uniform byte offsets
// into the packed and side arrays, or kOOB for a padding step.
template <int CODEC>
struct Raw;

template <>
struct Raw<0> {  // DYADIC: one bf16 scale per 64-group
  static constexpr uint32_t kPackedStep = 128;  // packed bytes per row and 256-k step
  static constexpr uint32_t kSideStep = 8;  // 4 groups x 2 bytes per 256-k step
  u32x4 a0, a1;
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.side, L.s + ss, 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable&, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const DyadicScale d = dyadic_scale(sb);
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
struct Raw<1> {  // LUT16: 16 bf16 levels (side) + bf16 scale (side2) per 64-group
  static constexpr uint32_t kPackedStep = 128;
  static constexpr uint32_t kSideStep = 128;  // 4 groups x 32 bytes
  u32x4 a0, a1, l0, l1;
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    const uint32_t loff = L.s + ss;
    l0 = __builtin_amdgcn_raw_buffer_load_b128(S.side, loff, 0, 0);
    l1 = __builtin_amdgcn_raw_buffer_load_b128(S.side, loff + 16, 0, 0);
    // scale offset = level offset / 16
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.side2, L.s2 + (ss == kOOB ? kOOB : ss >> 4), 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable&, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const Lut16Table t = lut16_table(sb, l0, l1);
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(j, lut16_rebuild(pw[j], t));
  }
};

template <>
struct Raw<2> {  // SIGNMAG8: two 32-groups, 8 fp16 magnitudes each
  static constexpr uint32_t kPackedStep = 128;
  static constexpr uint32_t kSideStep = 128;  // 8 groups x 16 bytes
  u32x4 a0, a1, c0, c1;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    const uint32_t coff = L.s + ss;
    c0 = __builtin_amdgcn_raw_buffer_load_b128(S.side, coff, 0, 0);
    c1 = __builtin_amdgcn_raw_buffer_load_b128(S.side, coff + 16, 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable&, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const SignMagTable t0 = signmag_table(c0), t1 = signmag_table(c1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 h, l;
      signmag_rebuild(pw[j], j < 4 ? t0 : t1, h, l);
      mma(j, h);
      mma(j, l);
    }
  }
};

template <>
struct Raw<3> {  // LUT16S: bf16 scale per 64-group; byte -> pair table (natural k order)
  static constexpr uint32_t kPackedStep = 128;
  static constexpr uint32_t kSideStep = 8;
  u32x4 a0, a1;
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.side, L.s + ss, 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable& st, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const float s = bf16_bits_to_f32(sb);
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(j, pair_rebuild(pw[j], s, st.tab));
  }
};

template <>
struct Raw<4> {  // DYADIC5: bf16 scale per 64-group (side) + high-bit words (side2)
  static constexpr uint32_t kPackedStep = 128;
  static constexpr uint32_t kSideStep = 8;  // 4 groups x 2 bytes per 256-k step
  u32x4 a0, a1;
  uint32_t h0, h1;  // high-bit words of the lane's two runs of 32 weights
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.side, L.s + ss, 0, 0);
    // 8 high-bit bytes per lane per step: offset step = 4 x the scale step
    const auto h = __builtin_amdgcn_raw_buffer_load_b64(S.side2, L.s2 + (ss == kOOB ? kOOB : 4 * ss),
                                                        0, 0);
    h0 = h[0];
    h1 = h[1];
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable&, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const Dyadic5Scale d = dyadic5_scale(sb);
    uint32_t e0, e1;
    if (__builtin_expect(__any(dyadic5_scale_is_wide(sb)), 0)) {
      const float pz = __builtin_bit_cast(float, opaque(0u));
#define W4_DYADIC5_STEP(J)                                         \
  dyadic5_msb<(J) & 3>((J) < 4 ? h0 : h1, e0, e1);                 \
  mma(J, dyadic5_rebuild(pw[J], e0, e1, d, pz));
      W4_DYADIC5_STEP(0)
      W4_DYADIC5_STEP(1)
      W4_DYADIC5_STEP(2)
      W4_DYADIC5_STEP(3)
      W4_DYADIC5_STEP(4)
      W4_DYADIC5_STEP(5)
      W4_DYADIC5_STEP(6)
      W4_DYADIC5_STEP(7)
#undef W4_DYADIC5_STEP
    } else {
#define W4_DYADIC5_STEP(J)                                         \
  dyadic5_msb<(J) & 3>((J) < 4 ? h0 : h1, e0, e1);                 \
  mma(J, dyadic5_rebuild_fma(pw[J], e0, e1, d));
      W4_DYADIC5_STEP(0)
      W4_DYADIC5_STEP(1)
      W4_DYADIC5_STEP(2)
      W4_DYADIC5_STEP(3)
      W4_DYADIC5_STEP(4)
      W4_DYADIC5_STEP(5)
      W4_DYADIC5_STEP(6)
      W4_DYADIC5_STEP(7)
#undef W4_DYADIC5_STEP
    }
  }
};

template <>
struct Raw<5> {  // LUT16S_PERM: LUT16S storage decoded by byte-plane v_perm lookups
  static constexpr uint32_t kPackedStep = 128;
  static constexpr uint32_t kSideStep = 8;  // 4 groups x 2 bytes per 256-k step
  u32x4 a0, a1;
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.side, L.s + ss, 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable& st, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const Lut16Table t = lut16_table(sb, st.l0, st.l1);
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(j, lut16_rebuild(pw[j], t));
  }
};

template <>
struct Raw<6> {  // LUT16S, scales interleaved into the packed records (side = packed)
  static constexpr uint32_t kPackedStep = kIlRecord;
  static constexpr uint32_t kSideStep = kIlRecord;
  u32x4 a0, a1;
  uint16_t sb;
  __device__ __forceinline__ void fetch(const Slice& S, const LaneBase& L, uint32_t sp,
                                        uint32_t ss) {
    a0 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pa + sp, 0, kPackedPolicy);
    a1 = __builtin_amdgcn_raw_buffer_load_b128(S.packed, L.pb + sp, 0, kPackedPolicy);
    sb = __builtin_amdgcn_raw_buffer_load_b16(S.packed, L.s + ss, 0, 0);
  }
  template <typename F>
  __device__ __forceinline__ void apply(const Shuffle& sh, const SharedTable& st, F&& mma) const {
    u32x4 p0, p1;
    sh(a0, a1, p0, p1);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const float s = bf16_bits_to_f32(sb);
#pragma unroll
    for (int j = 0; j < 8; ++j) mma(j, pair_rebuild(pw[j], s, st.tab));
  }
};

// k-chunk length staged in LDS for a given m and LDS capacity (16-byte units):
// rows of kc/8 units plus one pad unit each.
__host__ __device__ __forceinline__ int64_t gemv_chunk(int m, int xs_units, int64_t K) {
  int64_t kc = (int64_t)((xs_units / m - 1) / 32) * 256;
  const int64_t kpad = (K + 255) & ~(int64_t)255;
  return kc < kpad ? kc : kpad;
}

constexpr int kXFirst = 1;  // x units per thread loaded ahead of the weight prefetch

// k slices: for m > 1 a small matrix is also split along k across blocks
// (blockIdx.y = slice of slice_steps 256-k steps), so that every block stages
// only its slice's activations and the grid still fills the chip.  Each block
// then writes its fp32 partial sums to `part` [slice][m][n], and gemv_reduce
// adds the slices in order 0, 1, ... into y.  (A last-arriving block doing the
// sum instead would need a device-scope release per block, which on this chip
// writes back the whole L2 each time.)
struct Slicing {
  int kslices, slice_steps;
  float* part;
};

// XG: x units per thread kept in flight together while staging (after the
// first).  The batched m = 1 decode pass stages at most a few units per thread
// and runs fastest with the fewest registers, XG = 1; batched m >= 5 stages
// m x k activations per 64-row tile, as many bytes as the tile's weights at
// m = 16, and gains 6-11% from having all of a thread's units in flight at
// once, XG = 16; elsewhere XG = 4 (single calls' blocks of up to 1024 threads
// cannot spend the registers of a deeper staging).
template <int CODEC, int KSPLIT, bool BATCHED, int XG, bool RAGGED>
__global__ __launch_bounds__(64 * (KSPLIT > 4 ? KSPLIT : 4)) void gemv_kernel(
    GemvProblem single, const GemvProblem* probs, int count, int m, int y_bf16, int xs_units,
    Slicing sl) {
  constexpr int WAVES = KSPLIT > 4 ? KSPLIT : 4;
  constexpr int NT = 64 * WAVES;      // threads per block
  constexpr int RW = WAVES / KSPLIT;  // row tiles per block
  static_assert(!BATCHED || WAVES == 4, "the batched launch uses 4-wave blocks");
  // the pair decode yields weights in natural k order, so x is staged as is
  constexpr bool kNaturalX = CODEC == 3 || CODEC == 6;
  extern __shared__ u32x4 xs[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  GemvProblem P;
  int64_t blk = blockIdx.x;
  if constexpr (BATCHED) {
    // one round of parallel compares instead of a chain of dependent loads
    __shared__ int s_prob;
    if (tid == 0) s_prob = 0;
    __syncthreads();
    for (int t0 = 0; t0 < count; t0 += 256) {
      const int t = t0 + tid;
      if (t < count) {
        const int64_t b0 = probs[t].tile_begin;
        const int64_t b1 = b0 + (probs[t].n + RW * 16 - 1) / (RW * 16);
        if (b0 <= blk && blk < b1) s_prob = t;
      }
    }
    __syncthreads();
    P = probs[s_prob];
    blk -= P.tile_begin;
  } else {
    P = single;
  }
  const int64_t N = P.n, K = P.k;
  // this block's k range (whole rows unless sliced)
  int64_t kbeg = 0, kend = K;
  if constexpr (!BATCHED) {
    kbeg = (int64_t)blockIdx.y * sl.slice_steps * 256;
    const int64_t e = kbeg + (int64_t)sl.slice_steps * 256;
    kend = e < K ? e : K;
  }
  const int kw = wave % KSPLIT, rw = wave / KSPLIT;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t row0 = blk * RW * 16;
  const int rows_here = (int)((N - row0 < RW * 16) ? N - row0 : RW * 16);
  const uint32_t rloc = (uint32_t)(rw * 16 + r16);
  const int64_t row = row0 + rloc;
  const int mr = r16 < m ? r16 : m - 1;  // A row: batch row (padding rows repeat the last)
  // whole-line loads: lane = (row i of 8, chunk position cp); see Shuffle
  const int li = lane >> 3, cp = lane & 7;
  const uint32_t rowA = (uint32_t)(rw * 16 + li);
  const uint32_t chA = 16u * (uint32_t)(cp ^ ((li >> 1) & 7));
  const uint32_t chB = 16u * (uint32_t)(cp ^ (((li + 8) >> 1) & 7));
  Shuffle sh;
  sh.stage = xs + xs_units + 128 * wave;
  sh.wr = lane;
  {
    const int sw = (r16 >> 1) & 7;
    sh.rd0 = r16 * 8 + ((2 * q) ^ sw);
    sh.rd1 = r16 * 8 + ((2 * q + 1) ^ sw);
  }

  Slice S;
  constexpr bool kIL = CODEC == 6;
  // packed bytes of a row, and the packed offset of weight k0 (a multiple of 256)
  const uint32_t row_bytes = kIL ? (uint32_t)(K >> 8) * kIlRecord : (uint32_t)(K >> 1);
  auto pk_off = [&](int64_t kk) -> uint32_t {
    return kIL ? (uint32_t)(kk >> 8) * kIlRecord : (uint32_t)(kk >> 1);
  };
  const uint32_t g64 = (uint32_t)(K >> 6);  // 64-groups per row
  S.packed = rsrc(P.packed + (int64_t)row0 * row_bytes, (uint32_t)rows_here * row_bytes);
  if constexpr (kIL) {
    S.side = S.packed;
  } else if constexpr (CODEC == 0 || CODEC == 3 || CODEC == 5) {
    S.side = rsrc(P.scales + row0 * (K >> 6), (uint32_t)rows_here * g64 * 2);
  } else if constexpr (CODEC == 4) {
    S.side = rsrc(P.scales + row0 * (K >> 6), (uint32_t)rows_here * g64 * 2);
    S.side2 = rsrc(reinterpret_cast<const uint8_t*>(P.codebook) + row0 * (K >> 3),
                   (uint32_t)rows_here * (uint32_t)(K >> 3));
  } else if constexpr (CODEC == 1) {
    S.side = rsrc(P.codebook + row0 * (K >> 6) * 16, (uint32_t)rows_here * g64 * 32);
    S.side2 = rsrc(P.scales + row0 * (K >> 6), (uint32_t)rows_here * g64 * 2);
  } else {
    S.side = rsrc(P.codebook + row0 * (K >> 5) * 8, (uint32_t)rows_here * g64 * 32);
  }
  S.x = rsrc(P.x, (uint32_t)(m * K * 2));

  const int64_t kc = gemv_chunk(m, xs_units, kend - kbeg);
  // (a problem with k = 0 of a batch may pass no table: nothing reads it then)
  SharedTable st{};
  if constexpr (CODEC == 5) {
    if (K > 0) {
      st.l0 = reinterpret_cast<const u32x4*>(P.codebook)[0];
      st.l1 = reinterpret_cast<const u32x4*>(P.codebook)[1];
    }
  }
  if constexpr (CODEC == 3 || CODEC == 6) {
    // the pair table after the shuffle areas; written here, read after the
    // staging barrier of the first k-chunk
    f32x2* tab = reinterpret_cast<f32x2*>(xs + xs_units + 128 * WAVES);
    if (K > 0)
      for (int t = tid; t < 256; t += NT)
        tab[t] = (f32x2){bf16_bits_to_f32(P.codebook[t & 15]), bf16_bits_to_f32(P.codebook[t >> 4])};
    st.tab = tab;
  }
  const int row_units = (int)(kc / 8) + 1;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg; k0 < kend; k0 += kc) {
    const int64_t klen = (kend - k0 < kc) ? kend - k0 : kc;
    const int steps = (int)((klen + 255) >> 8);
    const int units = steps * 32;  // 16-byte units of one x row in this chunk
    // this wave's steps: st = kw + i * KSPLIT for i < nw; processed three at a
    // time, a padding step loads zeros (offset kOOB) and is not computed
    const int nw = steps > kw ? (steps - kw + KSPLIT - 1) / KSPLIT : 0;
    auto step_of = [&](int i) { return kw + i * KSPLIT; };
    LaneBase L;
    {
      const uint32_t g0 = rloc * g64 + (uint32_t)((k0 >> 6) + q);  // lane's first 64-group
      L.pa = rowA * row_bytes + pk_off(k0) + chA;
      L.pb = (rowA + 8) * row_bytes + pk_off(k0) + chB;
      L.s = kIL ? rloc * row_bytes + pk_off(k0) + 128u + 2u * (uint32_t)q
            : (CODEC == 0 || CODEC == 3 || CODEC == 4 || CODEC == 5) ? g0 * 2 : g0 * 32;
      L.s2 = CODEC == 4 ? rloc * (uint32_t)(K >> 3) + (uint32_t)(k0 >> 3) + 8u * (uint32_t)q
                        : g0 * 2;
    }
    // RAGGED: how far into the chunk each of the lane's loads starts; a load
    // of step st reads zeros unless 256 st + start < kend - k0
    uint32_t limA = 0, limB = 0, limS = 0;
    if constexpr (RAGGED) {
      const int64_t span = kend - k0;
      auto lim = [&](int64_t start) -> uint32_t {
        return span > start ? (uint32_t)(span - start) : 0u;
      };
      limA = lim(2 * (int64_t)chA);  // a 16-byte chunk holds 32 weights
      limB = lim(2 * (int64_t)chB);
      limS = lim(64 * (int64_t)q);    // the lane's 64-group of the step
    }
    auto fetch = [&](Raw<CODEC>& r, int i) {
      const bool in = i < nw;
      const uint32_t st = (uint32_t)step_of(i);
      if constexpr (RAGGED) {
        const uint32_t kst = 256u * st;
        LaneBase M;
        M.pa = opaque(kst < limA ? L.pa : kOOBLane);
        M.pb = opaque(kst < limB ? L.pb : kOOBLane);
        M.s = opaque(kst < limS ? L.s : kOOBLane);
        M.s2 = opaque(kst < limS ? L.s2 : kOOBLane);
        r.fetch(S, M, in ? st * Raw<CODEC>::kPackedStep : kOOB,
                in ? st * Raw<CODEC>::kSideStep : kOOB);
      } else {
        r.fetch(S, L, in ? st * Raw<CODEC>::kPackedStep : kOOB,
                in ? st * Raw<CODEC>::kSideStep : kOOB);
      }
    };
    // x staging slots: (row mrow, pass ip) -> unit tid + NT ip of that row
    const int ipr = (units + NT - 1) / NT;
    const int nslots = m * ipr;
    auto x_off = [&](int slot, int& mrow, int& uu) -> uint32_t {
      mrow = slot / ipr;  // uniform
      uu = tid + NT * (slot - mrow * ipr);
      const int64_t kk = k0 + 8 * (int64_t)uu;
      return (uu < units && kk < kend) ? (uint32_t)((mrow * K + kk) * 2) : kOOB;
    };
    lds_barrier();  // the previous chunk's LDS reads are done
    // activations first, then this wave's first three weight steps
    u32x4 xv[kXFirst];
    int xrow[kXFirst], xu[kXFirst];
#pragma unroll
    for (int i = 0; i < kXFirst; ++i) {
      const uint32_t o = x_off(i, xrow[i], xu[i]);
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(S.x, i < nslots ? o : kOOB, 0, 0);
    }
    // (issue order pinned: the loop's waits assume the buffers left in this order)
    Raw<CODEC> ra, rb, rc;
    __builtin_amdgcn_sched_barrier(0);
    fetch(ra, 0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(rb, 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(rc, 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kXFirst; ++i)
      if (i < nslots && xu[i] < units)
        xs[xrow[i] * row_units + xu[i]] = kNaturalX ? xv[i] : x_to_sigma(xv[i]);
    // the rest XG slots at a time, so their loads overlap
    for (int slot = kXFirst; slot < nslots; slot += XG) {
      u32x4 v[XG];
      int mrow[XG], uu[XG];
#pragma unroll
      for (int j = 0; j < XG; ++j) {
        const uint32_t o = x_off(slot + j, mrow[j], uu[j]);
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(S.x, slot + j < nslots ? o : kOOB, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < XG; ++j)
        if (slot + j < nslots && uu[j] < units)
          xs[mrow[j] * row_units + uu[j]] = kNaturalX ? v[j] : x_to_sigma(v[j]);
    }
    lds_barrier();

    auto compute = [&](const Raw<CODEC>& r, int i) {
      const u32x4* xa = &xs[mr * row_units + 32 * step_of(i) + 8 * q];
      r.apply(sh, st, [&](int j, const u32x4& b) { acc = mfma16x16x32(xa[j], b, acc); });
    };
    // three buffers in rotation: a buffer is refilled right after it is used,
    // so two steps stay in flight while one is computed and no live buffer is
    // ever copied (a copy would have to wait for its load)
    int i = 0;
    for (; i + 3 <= nw; i += 3) {  // the last one or two steps follow the loop
      compute(ra, i);
      fetch(ra, i + 3);
      compute(rb, i + 1);
      fetch(rb, i + 4);
      compute(rc, i + 2);
      fetch(rc, i + 5);
    }
    if (i < nw) compute(ra, i);
    if (i + 1 < nw) compute(rb, i + 1);
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

  if constexpr (KSPLIT == 1 && !BATCHED) {
    if (sl.kslices > 1) {
      if ((int)rloc >= rows_here) return;
      float* part = sl.part + (int64_t)blockIdx.y * m * N;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mrow = 4 * q + i;
        if (mrow < m) part[mrow * N + row] = acc[i];
      }
      return;
    }
  }

  if ((int)rloc >= rows_here) return;
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

// y[e] = sum over slices s = 0, 1, ... of part[s][e], e < total = m * n.
constexpr int kMaxSlices = 32;

__global__ __launch_bounds__(256) void gemv_reduce(const float* part, int kslices, int64_t total,
                                                   void* y, int y_bf16) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  // every slice's load in flight at once, then the sum in slice order
  float p[kMaxSlices];
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s) p[s] = s < kslices ? part[s * total + e] : 0.f;
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s)
    if (s < kslices) v += p[s];
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[e] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(y)[e] = v;
}

// y = +0 over `count` outputs (the product of an empty k range).
__global__ __launch_bounds__(256) void zero_kernel(void* y, int64_t count, int y_bf16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += stride) {
    if (y_bf16)
      reinterpret_cast<uint16_t*>(y)[e] = 0;
    else
      reinterpret_cast<float*>(y)[e] = 0.0f;
  }
}

// LDS units for a launch whose blocks each cover `kspan` of k: the whole
// padded span if it fits, else the cap; never less than the 1 KiB per wave
// the in-block k-split reduction needs.
// extra: LDS units the codec keeps after the shuffle areas (the pair table).
constexpr int extra_units(int codec) { return codec == 3 || codec == 6 ? 128 : 0; }

int xs_units_for(int m, int64_t kspan, int waves = 4, int extra = 0) {
  const int64_t kpad = (kspan + 255) & ~(int64_t)255;
  int64_t u = (int64_t)m * (kpad / 8 + 1);
  const int64_t cap = kLdsBlockUnits - 128 * waves - extra;
  if (u > cap) u = cap;
  if (u < 64 * waves) u = 64 * waves;
  return (int)u;
}

constexpr int kMaxSliceTiles = 1024;  // row tiles of a sliced call
constexpr int64_t kResidentWaves = 4096;  // 16 waves on each of 256 CUs
constexpr int64_t kTargetBlocks = 512;  // two blocks per CU

struct GemvShape {
  int ksplit;       // waves along k inside a block (1, 2, 4, 8, 16)
  int kslices;      // blocks along k
  int slice_steps;  // 256-k steps per slice
};

GemvShape gemv_shape(int64_t n, int64_t k, int m) {
  const int64_t steps = (k + 255) / 256;
  const int64_t tiles = (n + 63) / 64;
  if (m == 1 || tiles > kMaxSliceTiles) {
    // the activations of m = 1 are small: split k between the waves of a
    // block.  64-row tiles (4 waves, no split) while they give 1024 blocks,
    // else 32-row tiles; below that one 16-row tile per block whose 4, 8 or
    // 16 waves split k: the most waves per tile whose blocks all fit on the
    // GPU at once (these kernels keep 4 waves per SIMD, 16 per CU, resident;
    // a second round of blocks would cost more than the extra waves gain),
    // each wave keeping at least one 256-k step.
    int ks = 4;
    if (tiles >= 1024) {
      ks = 1;
    } else if ((n + 31) / 32 >= 1024) {
      ks = 2;
    } else {
      const int64_t tiles16 = (n + 15) / 16;
      while (ks < 16 && tiles16 * 2 * ks <= kResidentWaves && 2 * ks <= steps) ks *= 2;
    }
    if (m > 1) ks = 1;
    return {ks, 1, (int)steps};
  }
  // m >= 2 on few row tiles: when the whole m x k activations fit one
  // block's LDS, the same 16-row tiles with k split between the waves of a
  // block (one launch, partial sums added in LDS) beat k slices across
  // blocks and their second, reducing launch (measured: LUT16 4096^2 m = 4
  // 10.2 -> 7.5 us, 11008 x 4096 m = 2 16.4 -> 12.5 us, DYADIC 2048^2 m = 8
  // 8.3 -> 5.2 us).  The LDS bound keeps room for a decode table.
  {
    int ks = 4;
    const int64_t tiles16 = (n + 15) / 16;
    while (ks < 16 && tiles16 * 2 * ks <= kResidentWaves && 2 * ks <= steps) ks *= 2;
    auto fits = [&](int waves) {
      return m * (steps * 32 + 1) <= kLdsBlockUnits - 128 * (waves > 4 ? waves : 4) - 128;
    };
    while (ks > 4 && !fits(ks)) ks /= 2;
    if (fits(ks)) return {ks, 1, (int)steps};
  }
  // else the fewest slices whose activations fit in LDS, at least enough for
  // the grid
  int64_t fit = 1;
  while (fit < steps && m * (((steps + fit - 1) / fit) * 32 + 1) > kXsUnitsMax) ++fit;
  int64_t ks = (kTargetBlocks + tiles - 1) / tiles;
  if (ks < fit) ks = fit;
  if (ks > kMaxSlices) ks = kMaxSlices;
  if (ks > steps) ks = steps;
  if (ks < 1) ks = 1;  // k == 0 never gets here (the call writes zeros instead)
  const int64_t per = (steps + ks - 1) / ks;
  return {1, (int)((steps + per - 1) / per), (int)per};
}

template <int CODEC, int KSPLIT, bool RAGGED>
hipError_t launch_one(const GemvProblem& p, int m, int y_bf16, const GemvShape& sh,
                      hipStream_t stream) {
  constexpr int WAVES = KSPLIT > 4 ? KSPLIT : 4;
  const int rows = 16 * (WAVES / KSPLIT);
  const int64_t blocks = (p.n + rows - 1) / rows;
  Slicing sl{sh.kslices, sh.slice_steps, nullptr};
  if (sh.kslices > 1) {
    char* ws = nullptr;
    const hipError_t e =
        stream_workspace(kWorkspaceGemv, stream, (size_t)sh.kslices * m * p.n * 4, &ws);
    if (e != hipSuccess) return e;
    sl.part = reinterpret_cast<float*>(ws);
  }
  constexpr int EX = extra_units(CODEC);
  const int xu = xs_units_for(m, (int64_t)sh.slice_steps * 256, WAVES, EX);
  gemv_kernel<CODEC, KSPLIT, false, 4, RAGGED>
      <<<dim3((uint32_t)blocks, (uint32_t)sh.kslices), dim3(64 * WAVES),
         (xu + 128 * WAVES + EX) * 16, stream>>>(p, nullptr, 0, m, y_bf16, xu, sl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.kslices == 1) return e;
  const int64_t total = (int64_t)m * p.n;
  gemv_reduce<<<dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream>>>(
      sl.part, sh.kslices, total, p.y, y_bf16);
  return hipGetLastError();
}

template <int CODEC, bool RAGGED>
hipError_t launch_shape(const GemvProblem& p, int m, int y_bf16, const GemvShape& sh,
                        hipStream_t stream) {
  switch (sh.ksplit) {
    case 1: return launch_one<CODEC, 1, RAGGED>(p, m, y_bf16, sh, stream);
    case 2: return launch_one<CODEC, 2, RAGGED>(p, m, y_bf16, sh, stream);
    case 4: return launch_one<CODEC, 4, RAGGED>(p, m, y_bf16, sh, stream);
    case 8: return launch_one<CODEC, 8, RAGGED>(p, m, y_bf16, sh, stream);
    default: return launch_one<CODEC, 16, RAGGED>(p, m, y_bf16, sh, stream);
  }
}

// k slices and k chunks are whole 256-k steps, so only a k that is not a
// multiple of 256 leaves a partial last step.
template <int CODEC>
hipError_t launch_codec(const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  const GemvShape sh = gemv_shape(p.n, p.k, m);
  // (the interleaved layout holds whole 256-k records, so its k never is)
  if constexpr (CODEC != 6)
    if (p.k % 256) return launch_shape<CODEC, true>(p, m, y_bf16, sh, stream);
  return launch_shape<CODEC, false>(p, m, y_bf16, sh, stream);
}

}  // namespace

hipError_t launch_zero(void* y, int64_t count, int y_bf16, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  zero_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(y, count, y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemv(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream) {
  if (codec == 0) return launch_codec<0>(p, m, y_bf16, stream);
  if (codec == 1) return launch_codec<1>(p, m, y_bf16, stream);
  // LUT16S single calls decode per nibble: measured as fast as the byte ->
  // pair table or faster on every shape tried (2048^2 to 32768 x 4096, up
  // to 9% at 11008 x 4096), the table being built again by every block
  if (codec == 3 || codec == 5) return launch_codec<5>(p, m, y_bf16, stream);
  if (codec == 4) return launch_codec<4>(p, m, y_bf16, stream);
  if (codec == 6) return launch_codec<6>(p, m, y_bf16, stream);
  return launch_codec<2>(p, m, y_bf16, stream);
}

template <int CODEC, bool RAGGED>
hipError_t launch_batched_codec(const GemvProblem* probs_dev, int count, int64_t total_tiles,
                                int xu, int tile_rows, int m, int y_bf16, hipStream_t stream) {
  const dim3 block(256), grid((uint32_t)total_tiles);
  // activations + 4 x 2 KiB shuffle areas (+ the pair table)
  const size_t lds = (size_t)(xu + 512 + extra_units(CODEC)) * 16;
  const GemvProblem none{};
  const Slicing whole{1, 0, nullptr};
  // m == 1: tiles of 64 / 32 / 16 rows = 4 / 2 / 1 row tiles of 16 per block,
  // the block's 4 waves splitting k 1 / 2 / 4 ways
  if (m == 1 && tile_rows == 16)
    gemv_kernel<CODEC, 4, true, 1, RAGGED>
        <<<grid, block, lds, stream>>>(none, probs_dev, count, m, y_bf16, xu, whole);
  else if (m == 1 && tile_rows == 32)
    gemv_kernel<CODEC, 2, true, 1, RAGGED>
        <<<grid, block, lds, stream>>>(none, probs_dev, count, m, y_bf16, xu, whole);
  else if (m == 1)
    gemv_kernel<CODEC, 1, true, 1, RAGGED>
        <<<grid, block, lds, stream>>>(none, probs_dev, count, m, y_bf16, xu, whole);
  else if (m <= 4)  // (a deeper staging measured no faster at m <= 4 and slower at m = 2)
    gemv_kernel<CODEC, 1, true, 4, RAGGED>
        <<<grid, block, lds, stream>>>(none, probs_dev, count, m, y_bf16, xu, whole);
  else
    gemv_kernel<CODEC, 1, true, 16, RAGGED>
        <<<grid, block, lds, stream>>>(none, probs_dev, count, m, y_bf16, xu, whole);
  return hipGetLastError();
}

template <int CODEC>
hipError_t launch_batched_any(const GemvProblem* probs_dev, int count, int64_t total_tiles, int xu,
                              int tile_rows, int m, int y_bf16, bool ragged, hipStream_t stream) {
  if constexpr (CODEC == 6) {  // whole 256-k records: never ragged (checked by the caller)
    if (ragged) return hipErrorInvalidValue;
  } else if (ragged) {
    return launch_batched_codec<CODEC, true>(probs_dev, count, total_tiles, xu, tile_rows, m,
                                             y_bf16, stream);
  }
  return launch_batched_codec<CODEC, false>(probs_dev, count, total_tiles, xu, tile_rows, m,
                                            y_bf16, stream);
}

hipError_t launch_gemv_batched(int codec, const GemvProblem* probs_dev, int count,
                               int64_t total_tiles, int64_t k_max, int tile_rows, int m,
                               int y_bf16, bool ragged, hipStream_t stream) {
  // LUT16S: the byte -> pair table is built once per block, which pays on
  // 64-row tiles; the short tiles of a batch of a few large matrices decode
  // faster through the per-nibble lookups of the same storage (measured on
  // the three 3.9B-sized matrices: 18.4 against 22.4 us; the 168 decode-stack
  // matrices keep 64-row tiles, where the pair table is the faster one)
  if (codec == 3 && tile_rows < 64) codec = 5;
  const int xu = xs_units_for(m, k_max, 4, extra_units(codec));
  switch (codec) {
    case 5: return launch_batched_any<5>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    case 6: return launch_batched_any<6>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    case 0: return launch_batched_any<0>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    case 1: return launch_batched_any<1>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    case 3: return launch_batched_any<3>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    case 4: return launch_batched_any<4>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
    default: return launch_batched_any<2>(probs_dev, count, total_tiles, xu, tile_rows, m, y_bf16, ragged, stream);
  }
}

}  // namespace w4
