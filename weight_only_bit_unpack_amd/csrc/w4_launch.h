// Host-side launchers of the gfx950 kernels (internal to libw4; the public
// ABI is include/w4.h).  Arguments are validated by w4_api.cpp before any of
// these is called; each launcher only enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

// Same layout as w4_gemv_problem in include/w4.h.
struct GemvProblem {
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* codebook;
  const uint16_t* x;
  void* y;
  int64_t n;
  int64_t k;
  int64_t tile_begin;
};

hipError_t launch_quantize(int codec, int64_t n, int64_t k, const uint16_t* w, uint8_t* packed,
                           uint16_t* scales, const uint16_t* codebook, hipStream_t stream);

hipError_t launch_quantize_dyadic5(int64_t n, int64_t k, const uint16_t* w, const uint8_t* widths,
                                   uint8_t* packed, uint8_t* msb, uint16_t* scales,
                                   hipStream_t stream);

// W4_LUT16S_IL records (k a multiple of 256) from planar LUT16S arrays
hipError_t launch_lut16s_interleave(int64_t n, int64_t k, const uint8_t* packed,
                                    const uint16_t* scales, uint8_t* out, hipStream_t stream);

hipError_t launch_dequant(int codec, int64_t n, int64_t k, const uint8_t* packed,
                          const uint16_t* scales, const uint16_t* codebook, void* out,
                          hipStream_t stream);

hipError_t launch_lut16_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* scales,
                            uint16_t* lut, int iters, hipStream_t stream);
hipError_t launch_signmag8_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                               int iters, hipStream_t stream);
hipError_t launch_signmag8_warm_fit(int64_t n, int64_t k, const uint16_t* w, uint16_t* codebook,
                                    uint8_t* params, int iters, hipStream_t stream);

hipError_t launch_gemv(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream);

// y[0 .. count) = +0 (fp32, or bf16 when y_bf16): the product over k == 0.
hipError_t launch_zero(void* y, int64_t count, int y_bf16, hipStream_t stream);

// The batched GEMV's plan takes 64-row tiles, or for m == 1 halves them (down
// to 16) while the launch would have fewer than this many tiles.
constexpr int64_t kGemvBatchedMinTiles = 1024;
// probs_dev: count problems with tile_begin set by the plan for tiles of
// tile_rows (64; 32 or 16 only with m == 1) rows
// ragged: some problem's k is not a multiple of 256 (its last step is partial)
hipError_t launch_gemv_batched(int codec, const GemvProblem* probs_dev, int count,
                               int64_t total_tiles, int64_t k_max, int tile_rows, int m,
                               int y_bf16, bool ragged, hipStream_t stream);

// Library-owned device buffer of at least `bytes` for (current device, stream,
// user); its contents are undefined.  Growing allocates a new buffer and keeps
// the old one (work already enqueued, or a graph captured earlier, may still
// use it), so it never waits for the stream.
enum { kWorkspaceGemm = 0, kWorkspaceGemv = 1 };
hipError_t stream_workspace(int user, hipStream_t stream, size_t bytes, char** out);

// ws: a workspace of at least gemm_workspace_bytes(...) bytes, or nullptr for
// the library-kept one of the stream (stream_workspace)
hipError_t launch_gemm(int codec, const GemvProblem& p, int m, int y_bf16, hipStream_t stream,
                       char* ws);
size_t gemm_workspace_bytes(int codec, int64_t n, int64_t k, int m);

// Device address of the current device's copy of the fixed scratch array
// (w4_noalloc.hip), looked up once per device; its size in bytes.
hipError_t noalloc_scratch(char** out);
constexpr size_t kNoallocScratchBytes = size_t{64} << 20;

}  // namespace w4
