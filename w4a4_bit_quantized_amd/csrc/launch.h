// Internal kernel launchers of libw4a4 (not part of the public C ABI).
// Arguments are already validated by the entry points in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

// Activation (act = true: divide by smooth_factor, low-rank down-projection)
// or weight (act = false: multiply by smooth_factor) quantizer over `rows` x K.
// With parts > 1, K is split across workgroups and lora receives `parts`
// partial sums, each [rows, R], laid out one after another.
hipError_t launch_quantize(bool act, const void* x, const void* lam, const void* pd, int64_t rows, int64_t K,
                           int64_t R, int hadamard_block, int parts, void* q, void* scales, float* lora,
                           hipStream_t stream);

// Batches up to this many rows use the weight-streaming GEMM.
constexpr int64_t SKINNY_MAX_M = 32;

// Number of K parts the activation quantizer uses for svdq_linear at these sizes.
int quantize_parts(int64_t M, int64_t K);

// Block-scaled FP4 GEMM with the fused epilogue.  `lora` holds `lora_parts` partial sums,
// each [M, R], added in order (lora_parts > 1 only for batches of at most SKINNY_MAX_M rows).
hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, int lora_parts,
                       const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                       const void* wtscale, int64_t M, int64_t N, int64_t K, int64_t R, void* y, hipStream_t stream);

// Weight-streaming variant for M <= SKINNY_MAX_M (called by launch_gemm).
hipError_t launch_gemm_skinny(const void* qact, const void* ascales, const float* lora, int lora_parts,
                              const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                              const void* wtscale, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                              hipStream_t stream);

}  // namespace w4a4
