// C ABI of libw4 (declared in include/w4.h): argument validation on the host,
// then the kernel launches on the caller's stream.  Nothing is synchronised,
// and an error return leaves every buffer untouched.  The only allocation is
// the device workspace that w4_gemm and the m >= 2 GEMV keep per (device,
// stream) (w4_workspace.cpp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "w4.h"
#include "w4_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_codec(int32_t c) {
  return c == W4_DYADIC || c == W4_LUT16 || c == W4_SIGNMAG8 || c == W4_LUT16S ||
         c == W4_DYADIC5 || c == W4_LUT16S_PERM || c == W4_LUT16S_IL;
}

// W4_LUT16S_PERM shares LUT16S's storage and every kernel but the GEMV's.
int32_t storage_codec(int32_t c) { return c == W4_LUT16S_PERM ? W4_LUT16S : c; }

// Checks the quantized-weight triple of a codec for an [n][k] weight.  k must
// be a multiple of 64, or for SIGNMAG8 outside the matrix calls (whose kernels
// step over k in 64-weight units) of its group of 32.
w4_status check_weight(int32_t codec, int64_t n, int64_t k, const void* packed, const void* scales,
                       const void* codebook, bool matmul = false) {
  if (!valid_codec(codec)) return W4_EINVAL;
  if (n < 0 || k < 0) return W4_EINVAL;
  if (k % ((codec == W4_SIGNMAG8 && !matmul) ? 32 : 64)) return W4_ESHAPE;
  if (codec == W4_LUT16S_IL && k % 256) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!packed) return W4_EINVAL;
  if (!aligned(packed, 16)) return W4_EALIGN;
  codec = storage_codec(codec);
  if (codec == W4_DYADIC || codec == W4_LUT16 || codec == W4_LUT16S || codec == W4_DYADIC5) {
    if (!scales) return W4_EINVAL;
    if (!aligned(scales, 2)) return W4_EALIGN;
  }
  if (codec == W4_LUT16 || codec == W4_SIGNMAG8 || codec == W4_LUT16S || codec == W4_DYADIC5 ||
      codec == W4_LUT16S_IL) {
    if (!codebook) return W4_EINVAL;
    if (!aligned(codebook, 16)) return W4_EALIGN;
  }
  return W4_OK;
}

w4_status check_matmul(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                       const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                       int32_t m, void* y, int32_t y_dtype, int32_t m_max) {
  w4_status st = check_weight(codec, n, k, packed, scales, codebook, true);
  if (st != W4_OK) return st;
  if (m < 0) return W4_EINVAL;
  if (m > m_max) return W4_ESHAPE;
  if (y_dtype != W4_F32 && y_dtype != W4_BF16) return W4_EUNSUPPORTED;
  if (k > W4_MAX_MATMUL_K) return W4_ESHAPE;
  if (m == 0 || n == 0) return W4_OK;
  if (!y) return W4_EINVAL;
  if (!aligned(y, y_dtype == W4_F32 ? 4 : 2)) return W4_EALIGN;
  if (k > 0) {
    if (!x) return W4_EINVAL;
    if (!aligned(x, 16)) return W4_EALIGN;
  }
  return W4_OK;
}

w4_status launched(hipError_t e) { return e == hipSuccess ? W4_OK : W4_EHIP; }

w4::GemvProblem problem(int64_t n, int64_t k, const uint8_t* packed, const uint16_t* scales,
                        const uint16_t* codebook, const uint16_t* x, void* y) {
  w4::GemvProblem p;
  p.packed = packed;
  p.scales = scales;
  p.codebook = codebook;
  p.x = x;
  p.y = y;
  p.n = n;
  p.k = k;
  p.tile_begin = 0;
  return p;
}

constexpr int32_t kGemvMaxM = 16;
constexpr int32_t kGemmMaxM = 65535 * 128;

}  // namespace

static_assert(sizeof(w4_gemv_problem) == sizeof(w4::GemvProblem), "problem layout");
static_assert(sizeof(w4_gemv_batch_info) == 40, "batch info layout");
static_assert(W4_NOALLOC_SCRATCH_BYTES == w4::kNoallocScratchBytes, "scratch size");

extern "C" {

const char* w4_status_str(int32_t status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_EINVAL: return "W4_EINVAL: null pointer, bad enum or negative size";
    case W4_ESHAPE: return "W4_ESHAPE: k not a multiple of the group, m out of range, or too large";
    case W4_EALIGN: return "W4_EALIGN: pointer not aligned as required";
    case W4_EUNSUPPORTED: return "W4_EUNSUPPORTED: codec / dtype combination not provided";
    case W4_EHIP: return "W4_EHIP: kernel launch failed";
    default: return "unknown w4 status";
  }
}

int32_t w4_group_size(int32_t codec) {
  switch (codec) {
    case W4_DYADIC: return 64;
    case W4_LUT16: return 64;
    case W4_LUT16S: return 64;
    case W4_LUT16S_PERM: return 64;
    case W4_LUT16S_IL: return 64;
    case W4_DYADIC5: return 64;
    case W4_SIGNMAG8: return 32;
    default: return -1;
  }
}

w4_status w4_quantize_pack(int32_t codec, int64_t n, int64_t k, const uint16_t* w,
                           uint8_t* packed, uint16_t* scales, const uint16_t* codebook,
                           void* stream) {
  w4_status st = check_weight(codec, n, k, packed, scales, codebook);
  if (st != W4_OK) return st;
  if (codec == W4_DYADIC5 || codec == W4_LUT16S_IL) return W4_EUNSUPPORTED;
  if (n == 0 || k == 0) return W4_OK;
  if (!w) return W4_EINVAL;
  if (!aligned(w, 16)) return W4_EALIGN;
  return launched(w4::launch_quantize(storage_codec(codec), n, k, w, packed, scales, codebook,
                                      static_cast<hipStream_t>(stream)));
}

w4_status w4_unpack_dequant(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                            const uint16_t* scales, const uint16_t* codebook, void* out,
                            void* stream) {
  w4_status st = check_weight(codec, n, k, packed, scales, codebook);
  if (st != W4_OK) return st;
  if (codec == W4_LUT16S_IL) return W4_EUNSUPPORTED;
  if (n == 0 || k == 0) return W4_OK;
  if (!out) return W4_EINVAL;
  if (!aligned(out, 16)) return W4_EALIGN;
  return launched(w4::launch_dequant(storage_codec(codec), n, k, packed, scales, codebook, out,
                                     static_cast<hipStream_t>(stream)));
}

w4_status w4_lut16s_interleave(int64_t n, int64_t k, const uint8_t* packed, const uint16_t* scales,
                               uint8_t* out, void* stream) {
  if (n < 0 || k < 0) return W4_EINVAL;
  if (k % 256 != 0) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!packed || !scales || !out) return W4_EINVAL;
  if (!aligned(packed, 16) || !aligned(out, 16) || !aligned(scales, 2)) return W4_EALIGN;
  return launched(w4::launch_lut16s_interleave(n, k, packed, scales, out,
                                               static_cast<hipStream_t>(stream)));
}

w4_status w4_quantize_dyadic5(int64_t n, int64_t k, const uint16_t* w, const uint8_t* widths,
                              uint8_t* packed, uint8_t* msb, uint16_t* scales, void* stream) {
  if (n < 0 || k < 0) return W4_EINVAL;
  if (k % 64 != 0) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!w || !packed || !msb || !scales) return W4_EINVAL;
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(msb, 16) || !aligned(scales, 2))
    return W4_EALIGN;
  return launched(w4::launch_quantize_dyadic5(n, k, w, widths, packed, msb, scales,
                                              static_cast<hipStream_t>(stream)));
}

w4_status w4_lut16_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* scales,
                       uint16_t* codebook, int32_t iters, void* stream) {
  if (n < 0 || k < 0 || iters < 0 || iters > W4_MAX_FIT_ITERS) return W4_EINVAL;
  if (k % 64 != 0) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!w || !scales || !codebook) return W4_EINVAL;
  if (!aligned(w, 16) || !aligned(codebook, 16) || !aligned(scales, 2)) return W4_EALIGN;
  // one block per 16 groups: at most 2^31 - 1 blocks
  if (n > ((INT64_C(1) << 31) - 1) * 16 / (k / 64)) return W4_ESHAPE;
  return launched(w4::launch_lut16_fit(n, k, w, scales, codebook, iters,
                                       static_cast<hipStream_t>(stream)));
}

w4_status w4_signmag8_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                          int32_t iters, void* stream) {
  if (n < 0 || k < 0 || iters < 0 || iters > W4_MAX_FIT_ITERS) return W4_EINVAL;
  if (k % 32 != 0) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!w || !codebook) return W4_EINVAL;
  if (!aligned(w, 16) || !aligned(codebook, 16)) return W4_EALIGN;
  // one block per 32 groups: at most 2^31 - 1 blocks
  if (n > ((INT64_C(1) << 31) - 1) * 32 / (k / 32)) return W4_ESHAPE;
  return launched(w4::launch_signmag8_fit(n, k, w, codebook, iters,
                                          static_cast<hipStream_t>(stream)));
}

w4_status w4_signmag8_fit_warm(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                               uint8_t* params, int32_t iters, void* stream) {
  if (n < 0 || k < 0 || iters < 0 || iters > W4_MAX_FIT_ITERS) return W4_EINVAL;
  if (k % 32 != 0) return W4_ESHAPE;
  if (n == 0 || k == 0) return W4_OK;
  if (!w || !codebook) return W4_EINVAL;
  if (!aligned(w, 16) || !aligned(codebook, 16)) return W4_EALIGN;
  // one block per 2 groups: at most 2^31 - 1 blocks
  if (n > ((INT64_C(1) << 31) - 1) * 2 / (k / 32)) return W4_ESHAPE;
  return launched(w4::launch_signmag8_warm_fit(n, k, w, codebook, params, iters,
                                               static_cast<hipStream_t>(stream)));
}

w4_status w4_gemv(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                  const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                  int32_t m, void* y, int32_t y_dtype, void* stream) {
  w4_status st = check_matmul(codec, n, k, packed, scales, codebook, x, m, y, y_dtype, kGemvMaxM);
  if (st != W4_OK) return st;
  if (m == 0 || n == 0) return W4_OK;
  if (k == 0)  // the empty sum
    return launched(w4::launch_zero(y, (int64_t)m * n, y_dtype == W4_BF16,
                                    static_cast<hipStream_t>(stream)));
  return launched(w4::launch_gemv(codec, problem(n, k, packed, scales, codebook, x, y), m,
                                  y_dtype == W4_BF16, static_cast<hipStream_t>(stream)));
}

w4_status w4_gemm(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                  const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                  int32_t m, void* y, int32_t y_dtype, void* stream) {
  w4_status st = check_matmul(codec, n, k, packed, scales, codebook, x, m, y, y_dtype, kGemmMaxM);
  if (st != W4_OK) return st;
  if (codec == W4_LUT16S_IL) return W4_EUNSUPPORTED;
  if (m == 0 || n == 0) return W4_OK;
  if (k == 0)  // the empty sum
    return launched(w4::launch_zero(y, (int64_t)m * n, y_dtype == W4_BF16,
                                    static_cast<hipStream_t>(stream)));
  return launched(w4::launch_gemm(storage_codec(codec), problem(n, k, packed, scales, codebook, x, y),
                                  m, y_dtype == W4_BF16, static_cast<hipStream_t>(stream), nullptr));
}

w4_status w4_gemm_noalloc(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                          const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                          int32_t m, void* y, int32_t y_dtype, void* stream) {
  w4_status st = check_matmul(codec, n, k, packed, scales, codebook, x, m, y, y_dtype, kGemmMaxM);
  if (st != W4_OK) return st;
  if (codec == W4_LUT16S_IL) return W4_EUNSUPPORTED;
  if (m == 0 || n == 0) return W4_OK;
  if (k == 0)
    return launched(w4::launch_zero(y, (int64_t)m * n, y_dtype == W4_BF16,
                                    static_cast<hipStream_t>(stream)));
  codec = storage_codec(codec);
  if (w4::gemm_workspace_bytes(codec, n, k, m) > w4::kNoallocScratchBytes) return W4_ESHAPE;
  char* ws = nullptr;
  if (w4::noalloc_scratch(&ws) != hipSuccess) return W4_EHIP;
  return launched(w4::launch_gemm(codec, problem(n, k, packed, scales, codebook, x, y), m,
                                  y_dtype == W4_BF16, static_cast<hipStream_t>(stream), ws));
}

w4_status w4_linear(int32_t codec, int64_t n, int64_t k, const uint8_t* packed,
                    const uint16_t* scales, const uint16_t* codebook, const uint16_t* x,
                    int32_t m, void* y, int32_t y_dtype, void* stream) {
  if (m >= 0 && m <= kGemvMaxM)
    return w4_gemv(codec, n, k, packed, scales, codebook, x, m, y, y_dtype, stream);
  return w4_gemm(codec, n, k, packed, scales, codebook, x, m, y, y_dtype, stream);
}

w4_status w4_gemv_batched_plan(int32_t codec, int32_t m, int32_t y_dtype,
                               w4_gemv_problem* problems, int32_t count,
                               w4_gemv_batch_info* info) {
  if (!info || count < 0 || !problems) return W4_EINVAL;
  if (!valid_codec(codec)) return W4_EINVAL;
  if (m < 1) return m < 0 ? W4_EINVAL : W4_ESHAPE;
  for (int32_t i = 0; i < count; ++i) {
    const w4_gemv_problem& p = problems[i];
    w4_status st = check_matmul(codec, p.n, p.k, p.packed, p.scales, p.codebook, p.x, m, p.y,
                                y_dtype, kGemvMaxM);
    if (st != W4_OK) return st;
  }
  int64_t total = 0, kmax = 0, kmin = count > 0 ? problems[0].k : 0;
  for (int32_t i = 0; i < count; ++i) {
    if (problems[i].k > kmax) kmax = problems[i].k;
    if (problems[i].k < kmin) kmin = problems[i].k;
  }
  // the tallest tiles that still give the launch enough blocks
  auto tiles_of = [&](int64_t rows) {
    int64_t t = 0;
    for (int32_t i = 0; i < count; ++i) t += (problems[i].n + rows - 1) / rows;
    return t;
  };
  int64_t rows = 64;
  if (m == 1) {
    while (rows > 16 && tiles_of(rows) < w4::kGemvBatchedMinTiles) rows /= 2;
  }
  total = tiles_of(rows);
  if (total > 0x7FFFFFFF) return W4_ESHAPE;
  // Work is handed out in tile order; giving the longest rows (largest k) the
  // first tiles leaves short tiles for the end of the launch.
  std::vector<int32_t> order((size_t)count);
  for (int32_t i = 0; i < count; ++i) order[(size_t)i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return problems[a].k > problems[b].k; });
  total = 0;
  for (int32_t i : order) {
    problems[i].tile_begin = total;
    total += (problems[i].n + rows - 1) / rows;
  }
  info->total_tiles = total;
  info->k_min = kmin;
  info->k_max = kmax;
  info->count = count;
  info->m = m;
  info->tile_rows = (int32_t)rows;
  bool ragged = false;
  for (int32_t i = 0; i < count; ++i) ragged = ragged || (problems[i].k % 256 != 0);
  info->flags = ragged ? 1 : 0;
  return W4_OK;
}

w4_status w4_gemv_batched(int32_t codec, int32_t m, int32_t y_dtype,
                          w4_gemv_problem* problems_device, const w4_gemv_batch_info* info,
                          void* stream) {
  if (!info || !valid_codec(codec)) return W4_EINVAL;
  if (info->count < 0 || info->total_tiles < 0 || info->k_max < 0 || info->k_min < 0 ||
      (info->flags & ~1) != 0)
    return W4_EINVAL;
  if (info->m != m) return W4_EINVAL;  // the work numbering depends on m
  if (m < 1) return m < 0 ? W4_EINVAL : W4_ESHAPE;
  if (m > kGemvMaxM) return W4_ESHAPE;
  if (y_dtype != W4_F32 && y_dtype != W4_BF16) return W4_EUNSUPPORTED;
  // the interleaved layout needs every k a multiple of 256
  if (codec == W4_LUT16S_IL && (info->flags & 1)) return W4_ESHAPE;
  if (info->count == 0 || info->total_tiles == 0) return W4_OK;
  if (info->tile_rows != 64 && !(m == 1 && (info->tile_rows == 32 || info->tile_rows == 16)))
    return W4_EINVAL;
  if (!problems_device) return W4_EINVAL;
  if (!aligned(problems_device, 16)) return W4_EALIGN;
  if (info->total_tiles > 0x7FFFFFFF) return W4_ESHAPE;
  return launched(w4::launch_gemv_batched(
      codec, reinterpret_cast<const w4::GemvProblem*>(problems_device), info->count,
      info->total_tiles, info->k_max, info->tile_rows, m, y_dtype == W4_BF16,
      (info->flags & 1) != 0, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
