// The fixed scratch array of w4_gemm_noalloc (include/w4.h): a GEMM workspace
// that is never allocated at run time, for callers that cannot allocate.
//
// `scratch` is a file-scope device array of kNoallocScratchBytes; every GPU
// the library runs on holds its own copy until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for the symbol, not a
// device address: the device address of the current device's copy is looked
// up once per device with hipGetSymbolAddress and kept here, and only that
// address is ever passed to a kernel.
#include "w4_launch.h"

#include <map>
#include <mutex>

namespace w4 {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(char** out) {
  static std::mutex mu;
  static std::map<int, char*> addr;  // device -> address of its copy
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = addr.emplace(dev, static_cast<char*>(p)).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace w4
