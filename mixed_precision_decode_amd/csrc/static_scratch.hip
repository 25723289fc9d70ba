// Fixed device scratch for callers that cannot allocate (code under HIP
// graph capture, serving loops that forbid hipMalloc): the decode step's
// per-split partial results live in a file-scope device array instead of a
// caller workspace. Each device that the library runs on holds its own copy
// of the array, at its own address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace mikv {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
}  // namespace

// Device address of the current device's copy of `scratch`. The host-side
// name of the array is only a stand-in (a kernel handed it would fault), so
// the address is looked up once per device, with that device current, and
// kept; every later use goes through the kept pointer.
hipError_t static_scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_err[dev] = r;
    g_ptr[dev] = (r == hipSuccess) ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mikv
