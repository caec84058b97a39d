// Device scratch owned by the library for its allocation-free entry points
// (callers that cannot call hipMalloc: code under graph capture, serving
// loops, harnesses that forbid allocation).
//
// One file-scope device array of a fixed size.  Each GPU the library runs on
// holds its own copy at its own address until the process ends.  Host code
// never passes the array's name to a kernel or a copy (in host code the name
// is a host-side stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace sqattn {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

#ifdef SQATTN_DEBUG
static __device__ __align__(256) uint32_t violations[64];

hipError_t debug_word(uint32_t** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(violations));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = (uint32_t*)addr[dev];
  return hipSuccess;
}
#endif

}  // namespace sqattn
