// Library-owned device scratch for callers that cannot allocate (code under
// HIP graph capture, serving loops that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, from the moment the code object is loaded
// until the process ends.  In host code the name is only a stand-in for the
// symbol, not a device address, so host code never passes it to a kernel or a
// copy: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch_ptr.
#include <mutex>

#include "pkv_common.h"

namespace pkv {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
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

}  // namespace pkv
