// Internal kernel launchers of libw4a4 (not part of the public C ABI).
// Arguments are already validated by the entry points in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// Activation (act = true: divide by smooth_factor, low-rank down-projection)
// or weight (act = false: multiply by smooth_factor) quantizer over `rows` x K.
hipError_t launch_quantize(bool act, const void* x, const void* lam, const void* pd, int64_t rows, int64_t K,
                           int64_t R, int hadamard_block, void* q, void* scales, float* lora, hipStream_t stream);

// Block-scaled FP4 GEMM with the fused epilogue.
hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, const void* qweight,
                       const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                       int64_t M, int64_t N, int64_t K, int64_t R, void* y, hipStream_t stream);

}  // namespace w4a4
