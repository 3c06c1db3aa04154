// Device scratch of the no-allocation decode entry point.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the decode's
// cross-workgroup state from this file-scope array instead of a workspace
// argument.  Every GPU the library runs on holds its own copy of the array
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is a stand-in, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and cached.
#include <mutex>

#include "pkv_internal.hpp"

namespace pkv {

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device (NULL with the HIP error
// in *err when the lookup fails).  Called from the no-allocation entry point;
// the lookup runs once per device.
void* noalloc_scratch(hipError_t* err) {
  *err = hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace pkv
