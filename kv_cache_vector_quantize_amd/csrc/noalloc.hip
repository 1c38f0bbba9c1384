// Device scratch of the allocation-free decode entry point: a fixed array in
// the library's code object, one copy per device, held until the process
// ends.  Its device address is looked up once per device (with that device
// current) and cached; host code uses only that address, never the array's
// name (which on the host is a stand-in, not a device address).
#include <mutex>

#include "tq_internal.hpp"

namespace tq {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
