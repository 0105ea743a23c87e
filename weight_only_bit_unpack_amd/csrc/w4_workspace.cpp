// Device workspaces kept by the library per (device, stream, user).
//
// A matrix-product call that needs scratch memory (packed activations, k-split
// partial sums) takes it from here: the buffer is allocated on first use and
// replaced by a larger one when a call needs more.  A replaced buffer is
// never freed: kernels enqueued earlier on the stream, and HIP graphs captured
// earlier, may still read and write it, and freeing it would need a wait for
// the stream.  Each replacement at least doubles the size, so the buffers a
// (device, stream, user) ever holds add up to less than twice the largest.
// Calls on one stream are ordered and share the current buffer; calls on
// different streams never share one.  Nothing is released before the process
// ends, also for streams the caller has destroyed.
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
    size_t want = bytes;
    if (want < 2 * slot.second) want = 2 * slot.second;
    char* p = nullptr;
    e = hipMalloc(reinterpret_cast<void**>(&p), want);
    if (e != hipSuccess) return e;
    slot = {p, want};  // the old buffer stays allocated (see above)
  }
  *out = slot.first;
  return hipSuccess;
}

}  // namespace w4
