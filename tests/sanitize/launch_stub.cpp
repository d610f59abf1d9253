// Host-only stand-ins for the kernel launchers and the one HIP runtime call of the C-ABI layer,
// for the AddressSanitizer / UndefinedBehaviorSanitizer build of the host code (api.cpp and
// lowrank_split.cpp).  That build runs on a machine without a GPU and exercises only argument
// validation and the host-side offline split: every launcher reports that no device is present,
// so a call that passes validation returns W4A4_ERR_HIP without touching device memory.
#include <hip/hip_runtime_api.h>

#include "launch.h"

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace w4a4 {

hipError_t launch_quantize(bool, const void*, const void*, const void*, int64_t, int64_t, int64_t, int, int, void*,
                           void*, float*, hipStream_t, bool, int64_t) {
  return hipErrorNoDevice;
}

hipError_t launch_gemm(const void*, const void*, const float*, int, const void*, const void*, const void*, const void*,
                       const void*, const void*, int64_t, int64_t, int64_t, int64_t, void*, hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_gemm_mx(const void*, const void*, const float*, int, const void*, const void*, const void*,
                          const void*, const void*, const void*, int64_t, int64_t, int64_t, int64_t, int64_t, void*,
                          hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_gemm_skinny(const void*, const void*, const float*, int, const void*, const void*, const void*,
                              const void*, const void*, const void*, int64_t, int64_t, int64_t, int64_t, void*,
                              hipStream_t) {
  return hipErrorNoDevice;
}

hipError_t launch_hadamard(const void*, int64_t, void*, int64_t, int64_t, int64_t, int, int, float, hipStream_t) {
  return hipErrorNoDevice;
}

void* noalloc_scratch() { return nullptr; }

}  // namespace w4a4
