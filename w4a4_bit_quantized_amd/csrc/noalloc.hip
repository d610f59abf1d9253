// The static device workspace of svdq_linear_noalloc (the entry point itself is in api.cpp): the
// whole layer for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The kernels are svdq_linear's; only the
// workspace's home differs.
//
// `scratch` is a file-scope device array.  Host code never uses its name as an address (on the
// host the name is only a stand-in): the device address is fetched once per device with
// hipGetSymbolAddress while that device is current, kept per device, and passed to the kernels as
// svdq_linear's workspace.  Each GPU holds its own copy until the process ends; every call on a
// GPU shares it, so calls that overlap on one GPU race.  The workspace needs no initialisation
// (every byte the kernels read is written earlier in the same call), so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "w4a4.h"

namespace {

__device__ __align__(256) uint8_t scratch[W4A4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

}  // namespace

namespace w4a4 {

// Device address of `scratch` on the current device (looked up once per device, with that device
// current), or NULL if the lookup failed.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceScratch& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  return s.err == hipSuccess ? s.ptr : nullptr;
}

}  // namespace w4a4
