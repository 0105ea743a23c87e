// Device workspaces kept by the library per (device, stream, user).
//
// A matrix-product call that needs scratch memory (packed activations, k-split
// partial sums) takes it from here: the buffer is allocated
// on first use, grown when a call needs more, and kept until the process ends,
// so later calls only enqueue kernels.  Calls on one stream are ordered and
// may share a buffer; calls on different streams never do.
#include "w4_launch.h"

#include <map>
#include <mutex>
#include <tuple>

namespace w4 {

hipError_t stream_workspace(int user, hipStream_t stream, size_t bytes, char** out) {
  static std::mutex mu;
  static std::map<std::tuple<int, hipStream_t, int>, std::pair<char*, size_t>> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  auto& slot = cache[std::make_tuple(dev, stream, user)];
  if (slot.second < bytes) {
    if (slot.first) {
      // the stream may still be using the old buffer
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return e;
      e = hipFree(slot.first);
      if (e != hipSuccess) return e;
      slot = {nullptr, 0};
    }
    char* p = nullptr;
    e = hipMalloc(reinterpret_cast<void**>(&p), bytes);
    if (e != hipSuccess) return e;
    slot = {p, bytes};
  }
  *out = slot.first;
  return hipSuccess;
}

}  // namespace w4
