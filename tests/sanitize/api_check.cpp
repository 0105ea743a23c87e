// Host-side check of the C ABI's argument validation and batched planning
// (w4_api.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the CPU.  The kernel launchers are replaced by stubs that record what they
// were asked to do, so every path of the validation layer runs without a
// GPU.  Test infrastructure: built and run by tests/test_sanitize.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "w4.h"
#include "w4_launch.h"

namespace {
int g_launches = 0;
int g_last_codec = -1;
int64_t g_last_count = -1;
bool g_last_ragged = false;
size_t g_workspace = 0;
char g_scratch[256];
}  // namespace

namespace w4 {
hipError_t launch_quantize(int codec, int64_t, int64_t, const uint16_t*, uint8_t*, uint16_t*,
                           const uint16_t*, hipStream_t) {
  ++g_launches;
  g_last_codec = codec;
  return hipSuccess;
}
hipError_t launch_quantize_dyadic5(int64_t, int64_t, const uint16_t*, const uint8_t*, uint8_t*,
                                   uint8_t*, uint16_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_lut16s_interleave(int64_t, int64_t, const uint8_t*, const uint16_t*, uint8_t*,
                                    hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dequant(int codec, int64_t, int64_t, const uint8_t*, const uint16_t*,
                          const uint16_t*, void*, hipStream_t) {
  ++g_launches;
  g_last_codec = codec;
  return hipSuccess;
}
hipError_t launch_lut16_fit(int64_t, int64_t, const uint16_t*, uint16_t*, uint16_t*, int,
                            hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_signmag8_fit(int64_t, int64_t, const uint16_t*, uint16_t*, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_signmag8_warm_fit(int64_t, int64_t, const uint16_t*, uint16_t*, uint8_t*, int,
                                    hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gemv(int codec, const GemvProblem&, int, int, hipStream_t) {
  ++g_launches;
  g_last_codec = codec;
  return hipSuccess;
}
hipError_t launch_zero(void*, int64_t count, int, hipStream_t) {
  ++g_launches;
  g_last_codec = -2;
  g_last_count = count;
  return hipSuccess;
}
hipError_t launch_gemv_batched(int codec, const GemvProblem*, int count, int64_t, int64_t, int,
                               int, int, bool ragged, hipStream_t) {
  ++g_launches;
  g_last_codec = codec;
  g_last_count = count;
  g_last_ragged = ragged;
  return hipSuccess;
}
hipError_t launch_gemm(int codec, const GemvProblem&, int, int, hipStream_t, char*) {
  ++g_launches;
  g_last_codec = codec;
  return hipSuccess;
}
size_t gemm_workspace_bytes(int, int64_t, int64_t, int) { return g_workspace; }
hipError_t noalloc_scratch(char** out) {
  *out = g_scratch;
  return hipSuccess;
}
}  // namespace w4

namespace {
int failures = 0;
void expect(bool ok, const char* what, int line) {
  if (!ok) {
    fprintf(stderr, "FAIL line %d: %s\n", line, what);
    ++failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// 16-byte aligned fake device addresses (never dereferenced by the stubs)
uint8_t* P(uintptr_t a) { return reinterpret_cast<uint8_t*>(a); }
uint16_t* H(uintptr_t a) { return reinterpret_cast<uint16_t*>(a); }
}  // namespace

int main() {
  const uintptr_t A = 0x10000;
  // --- quantize / dequant
  int before = g_launches;
  EXPECT(w4_quantize_pack(0, 4, 64, H(A), P(A), H(A), nullptr, nullptr) == W4_OK);
  EXPECT(g_launches == before + 1 && g_last_codec == 0);
  EXPECT(w4_quantize_pack(5, 4, 64, H(A), P(A), H(A), H(A), nullptr) == W4_OK);
  EXPECT(g_last_codec == W4_LUT16S);  // PERM quantizes as LUT16S
  EXPECT(w4_quantize_pack(0, 4, 96, H(A), P(A), H(A), nullptr, nullptr) == W4_ESHAPE);
  EXPECT(w4_quantize_pack(2, 4, 96, H(A), P(A), nullptr, H(A), nullptr) == W4_OK);
  EXPECT(w4_quantize_pack(2, 4, 80, H(A), P(A), nullptr, H(A), nullptr) == W4_ESHAPE);
  EXPECT(w4_quantize_pack(4, 4, 64, H(A), P(A), H(A), H(A), nullptr) == W4_EUNSUPPORTED);
  EXPECT(w4_quantize_pack(6, 4, 256, H(A), P(A), nullptr, H(A), nullptr) == W4_EUNSUPPORTED);
  EXPECT(w4_quantize_pack(7, 4, 64, H(A), P(A), H(A), H(A), nullptr) == W4_EINVAL);
  EXPECT(w4_quantize_pack(0, -1, 64, H(A), P(A), H(A), nullptr, nullptr) == W4_EINVAL);
  EXPECT(w4_quantize_pack(0, 4, 64, H(A + 2), P(A), H(A), nullptr, nullptr) == W4_EALIGN);
  EXPECT(w4_quantize_pack(0, 4, 64, nullptr, P(A), H(A), nullptr, nullptr) == W4_EINVAL);
  before = g_launches;
  EXPECT(w4_quantize_pack(0, 0, 64, nullptr, nullptr, nullptr, nullptr, nullptr) == W4_OK);
  EXPECT(g_launches == before);
  EXPECT(w4_unpack_dequant(5, 4, 64, P(A), H(A), H(A), P(A), nullptr) == W4_OK);
  EXPECT(g_last_codec == W4_LUT16S);
  EXPECT(w4_unpack_dequant(6, 4, 256, P(A), nullptr, H(A), P(A), nullptr) == W4_EUNSUPPORTED);
  EXPECT(w4_unpack_dequant(0, 4, 64, P(A), H(A), nullptr, P(A + 8), nullptr) == W4_EALIGN);
  EXPECT(w4_lut16s_interleave(4, 256, P(A), H(A), P(A), nullptr) == W4_OK);
  EXPECT(w4_lut16s_interleave(4, 320, P(A), H(A), P(A), nullptr) == W4_ESHAPE);
  EXPECT(w4_quantize_dyadic5(4, 64, H(A), nullptr, P(A), P(A), H(A), nullptr) == W4_OK);
  EXPECT(w4_lut16_fit(4, 64, H(A), H(A), H(A), W4_MAX_FIT_ITERS + 1, nullptr) == W4_EINVAL);
  EXPECT(w4_signmag8_fit(4, 32, H(A), H(A), 25, nullptr) == W4_OK);
  EXPECT(w4_signmag8_fit_warm(4, 48, H(A), H(A), nullptr, 25, nullptr) == W4_ESHAPE);

  // --- matrix calls
  EXPECT(w4_gemv(0, 16, 64, P(A), H(A), nullptr, H(A), 1, P(A), W4_F32, nullptr) == W4_OK);
  EXPECT(w4_gemv(0, 16, 64, P(A), H(A), nullptr, H(A), 17, P(A), W4_F32, nullptr) == W4_ESHAPE);
  EXPECT(w4_gemv(0, 16, 64, P(A), H(A), nullptr, H(A), 1, P(A), W4_F16, nullptr) ==
         W4_EUNSUPPORTED);
  EXPECT(w4_gemv(2, 16, 96, P(A), nullptr, H(A), H(A), 1, P(A), W4_F32, nullptr) == W4_ESHAPE);
  EXPECT(w4_gemv(0, 16, W4_MAX_MATMUL_K + 64, P(A), H(A), nullptr, H(A), 1, P(A), W4_F32,
                 nullptr) == W4_ESHAPE);
  EXPECT(w4_gemv(0, 16, 0, nullptr, nullptr, nullptr, nullptr, 3, P(A), W4_F32, nullptr) == W4_OK);
  EXPECT(g_last_codec == -2 && g_last_count == 48);  // k = 0: zeros
  EXPECT(w4_gemm(5, 16, 64, P(A), H(A), H(A), H(A), 300, P(A), W4_BF16, nullptr) == W4_OK);
  EXPECT(g_last_codec == W4_LUT16S);
  EXPECT(w4_gemm(6, 16, 256, P(A), nullptr, H(A), H(A), 300, P(A), W4_F32, nullptr) ==
         W4_EUNSUPPORTED);
  EXPECT(w4_gemv(6, 16, 256, P(A), nullptr, H(A), H(A), 2, P(A), W4_F32, nullptr) == W4_OK);
  EXPECT(g_last_codec == W4_LUT16S_IL);
  g_workspace = (size_t)W4_NOALLOC_SCRATCH_BYTES + 1;
  EXPECT(w4_gemm_noalloc(0, 16, 64, P(A), H(A), nullptr, H(A), 300, P(A), W4_F32, nullptr) ==
         W4_ESHAPE);
  g_workspace = 1024;
  EXPECT(w4_gemm_noalloc(0, 16, 64, P(A), H(A), nullptr, H(A), 300, P(A), W4_F32, nullptr) ==
         W4_OK);
  EXPECT(w4_linear(0, 16, 64, P(A), H(A), nullptr, H(A), 16, P(A), W4_F32, nullptr) == W4_OK);

  // --- batched plan: random problems, then the plan's invariants
  srand(7);
  for (int trial = 0; trial < 200; ++trial) {
    const int count = 1 + rand() % 300;
    const int m = trial % 3 == 0 ? 1 + rand() % 16 : 1;
    std::vector<w4_gemv_problem> probs((size_t)count);
    bool ragged = false;
    for (int i = 0; i < count; ++i) {
      w4_gemv_problem& p = probs[(size_t)i];
      p.packed = P(A);
      p.scales = H(A);
      p.codebook = nullptr;
      p.x = H(A);
      p.y = P(A);
      p.n = rand() % 5 == 0 ? 0 : 1 + rand() % 5000;
      p.k = 64 * (1 + rand() % 100);
      p.tile_begin = -12345;
      ragged = ragged || (p.k % 256 != 0);
    }
    w4_gemv_batch_info info{};
    EXPECT(w4_gemv_batched_plan(0, m, W4_F32, probs.data(), count, &info) == W4_OK);
    EXPECT(info.count == count && info.m == m && info.flags == (ragged ? 1 : 0));
    EXPECT(info.tile_rows == 64 || (m == 1 && (info.tile_rows == 32 || info.tile_rows == 16)));
    // tiles: disjoint ranges that cover [0, total), larger k first
    std::vector<int64_t> owner((size_t)info.total_tiles, -1);
    for (int i = 0; i < count; ++i) {
      const w4_gemv_problem& p = probs[(size_t)i];
      const int64_t t = (p.n + info.tile_rows - 1) / info.tile_rows;
      EXPECT(p.tile_begin >= 0 && p.tile_begin + t <= info.total_tiles);
      for (int64_t j = 0; j < t; ++j) {
        if (p.tile_begin + j >= 0 && p.tile_begin + j < info.total_tiles) {
          EXPECT(owner[(size_t)(p.tile_begin + j)] == -1);
          owner[(size_t)(p.tile_begin + j)] = i;
        }
      }
    }
    int64_t prev_k = INT64_MAX;
    for (int64_t t = 0; t < info.total_tiles; ++t) {
      EXPECT(owner[(size_t)t] >= 0);
      if (owner[(size_t)t] >= 0) {
        const int64_t k = probs[(size_t)owner[(size_t)t]].k;
        EXPECT(k <= prev_k);
        prev_k = k;
      }
    }
    before = g_launches;
    EXPECT(w4_gemv_batched(0, m, W4_F32, reinterpret_cast<w4_gemv_problem*>(A), &info, nullptr) ==
           (info.total_tiles > 0 ? W4_OK : W4_OK));
    if (info.total_tiles > 0) EXPECT(g_launches == before + 1 && g_last_ragged == ragged);
  }
  w4_gemv_problem bad{};
  bad.packed = P(A);
  bad.scales = H(A);
  bad.x = H(A);
  bad.y = P(A);
  bad.n = 8;
  bad.k = 96;
  w4_gemv_batch_info info{};
  EXPECT(w4_gemv_batched_plan(0, 1, W4_F32, &bad, 1, &info) == W4_ESHAPE);
  info.flags = 2;
  EXPECT(w4_gemv_batched(0, 1, W4_F32, reinterpret_cast<w4_gemv_problem*>(A), &info, nullptr) ==
         W4_EINVAL);
  for (int s = -1; s < 8; ++s) EXPECT(w4_status_str(s) != nullptr);

  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("api_check ok\n");
  return 0;
}
