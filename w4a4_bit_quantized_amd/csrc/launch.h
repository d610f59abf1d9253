// Internal kernel launchers of libw4a4 (not part of the public C ABI).
// Arguments are already validated by the entry points in api.cpp.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>

namespace w4a4 {

// Kernel-path overrides.  Only the test build of the library (compiled with W4A4_TEST_HOOKS)
// reads them, from the environment, so that tests can force every kernel variant; in the
// product build every hook is absent and the automatic choice always applies.
#ifdef W4A4_TEST_HOOKS
inline const char* test_hook(const char* name) { return getenv(name); }
#else
inline const char* test_hook(const char*) { return nullptr; }
#endif

// Activation (act = true: divide by smooth_factor, low-rank down-projection)
// or weight (act = false: multiply by smooth_factor) quantizer over `rows` x K.
// With parts > 1, K is split across workgroups and lora receives `parts`
// partial sums, each [rows, R], laid out one after another.
// With mx, the scales are MXFP4 E8M0 bytes per 32 columns in rows of scale_stride bytes
// (scale_stride >= rows; entries rows .. scale_stride - 1 receive 0) and hadamard_block is 0 or 32.
hipError_t launch_quantize(bool act, const void* x, const void* lam, const void* pd, int64_t rows, int64_t K,
                           int64_t R, int hadamard_block, int parts, void* q, void* scales, float* lora,
                           hipStream_t stream, bool mx = false, int64_t scale_stride = 0);

// Batches up to this many rows use the weight-streaming GEMM.
constexpr int64_t SKINNY_MAX_M = 32;

// Number of K parts the activation quantizer uses for svdq_linear at these sizes.
int quantize_parts(int64_t M, int64_t K);

// Block-scaled FP4 GEMM with the fused epilogue.  `lora` holds `lora_parts` partial sums,
// each [M, R], added in order (lora_parts > 1 only for batches of at most SKINNY_MAX_M rows).
// `bias` (bf16 [N]) may be null.
hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, int lora_parts,
                       const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                       const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                       hipStream_t stream);

// MXFP4 GEMM (E8M0 scales per 32 columns; K % 128 == 0, N % 4 == 0; the activation scales
// are (K/32, ms) with ms = M rounded up to 4) with the same fused epilogue.
hipError_t launch_gemm_mx(const void* qact, const void* ascales, const float* lora, int lora_parts,
                          const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                          const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                          int64_t ms, void* y, hipStream_t stream);

// Weight-streaming variant for M <= SKINNY_MAX_M (called by launch_gemm).
hipError_t launch_gemm_skinny(const void* qact, const void* ascales, const float* lora, int lora_parts,
                              const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                              const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                              void* y, hipStream_t stream);

// MXFP4 weight-streaming variant for M <= 16, K <= 5120 a multiple of 512, R <= 64, at most 8
// low-rank parts (called by launch_gemm_mx; `ms` is the activation scale row stride).
bool skinny_mx_supported(int64_t M, int64_t K, int64_t R, int lora_parts);
hipError_t launch_gemm_skinny_mx(const void* qact, const void* ascales, const float* lora, int lora_parts,
                                 const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                                 const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                 int64_t ms, void* y, hipStream_t stream);

// Standalone block Hadamard transform of rows x cols elements (row strides ldx, ldy in
// elements; dtype 0 bf16, 1 f16, 2 f32; block a power of two in [2, 4096] dividing cols);
// norm = float32(1 / sqrt(block)).  x == y (with ldx == ldy) transforms in place.
hipError_t launch_hadamard(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols, int block,
                           int dtype, float norm, hipStream_t stream);

// Device address of the static workspace of svdq_linear_noalloc on the current device (looked up
// once per device), or NULL when the lookup fails.
void* noalloc_scratch();

}  // namespace w4a4
