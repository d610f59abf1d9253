// C-ABI entry points of libw4a4: argument validation, then kernel launches.
// The contract of each entry point is documented in include/w4a4.h.
#include "w4a4.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;  // sizes are indexed with 32-bit ints in the kernels
constexpr int64_t kMaxK = W4A4_MAX_K;     // tile-local byte offsets (rows x K/2) are 32-bit

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

w4a4_status check_k_rank_block(int64_t K, int64_t R, int32_t hb) {
  if (hb != 0 && hb != 16 && hb != 32 && hb != 64 && hb != 128) return W4A4_ERR_UNSUPPORTED;
  if (R > W4A4_MAX_RANK || K > kMaxK) return W4A4_ERR_UNSUPPORTED;
  if (K < 16 || K % 16 != 0 || K > kMaxDim || R < 0) return W4A4_ERR_SHAPE;
  if (hb != 0 && K % hb != 0) return W4A4_ERR_SHAPE;
  return W4A4_OK;
}

w4a4_status from_hip(hipError_t e) { return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP; }

// Order of checks everywhere: sizes, then the empty call (M or N == 0: valid, launches
// nothing, pointers may be NULL), then NULL pointers, then alignment.
w4a4_status validate_quantize_act(const void* x, const void* lam, const void* pd, int64_t M, int64_t K, int64_t R,
                                  int32_t hb, const void* qact, const void* ascales, const float* lora) {
  w4a4_status st = check_k_rank_block(K, R, hb);
  if (st != W4A4_OK) return st;
  if (M < 0 || M > kMaxDim) return W4A4_ERR_SHAPE;
  if (M == 0) return W4A4_OK;
  if (!x || !lam || !qact || !ascales) return W4A4_ERR_NULL;
  if (R > 0 && (!pd || !lora)) return W4A4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(lam, 16) || !aligned(qact, 4)) return W4A4_ERR_ALIGN;
  if (R > 0 && (!aligned(pd, 2) || !aligned(lora, 4))) return W4A4_ERR_ALIGN;
  return W4A4_OK;
}

w4a4_status validate_gemm(const void* qact, const void* ascales, const float* lora, const void* qweight,
                          const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                          int64_t M, int64_t N, int64_t K, int64_t R, const void* y) {
  w4a4_status st = check_k_rank_block(K, R, 0);
  if (st != W4A4_OK) return st;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return W4A4_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return W4A4_ERR_SHAPE;  // 1-D grid of output tiles
  if (M == 0 || N == 0) return W4A4_OK;
  if (!qact || !ascales || !qweight || !wscales || !wcscales || !wtscale || !y) return W4A4_ERR_NULL;
  if (R > 0 && (!lora || !proj_up)) return W4A4_ERR_NULL;
  if (!aligned(qact, 16) || !aligned(qweight, 16)) return W4A4_ERR_ALIGN;
  if (!aligned(wcscales, 2) || !aligned(wtscale, 2) || !aligned(y, 2)) return W4A4_ERR_ALIGN;
  if (R > 0 && (!aligned(lora, 4) || !aligned(proj_up, 2))) return W4A4_ERR_ALIGN;
  return W4A4_OK;
}

}  // namespace

namespace w4a4 {

int quantize_parts(int64_t M, int64_t K) {
  // Small batches split K across workgroups so that enough CUs stream x; the partial
  // low-rank sums are added in a fixed order by the consumer.
  const int64_t n64 = K / 64;
  if (M > SKINNY_MAX_M || n64 < 16) return 1;
  return (int)(n64 / 8 < 8 ? n64 / 8 : 8);
}

}  // namespace w4a4

extern "C" {

const char* w4a4_status_string(int status) {
  switch (status) {
    case W4A4_OK: return "ok";
    case W4A4_ERR_NULL: return "a required pointer is NULL";
    case W4A4_ERR_SHAPE: return "invalid sizes (negative, K % 16 != 0, K % hadamard_block != 0, or workspace too small)";
    case W4A4_ERR_ALIGN: return "a pointer breaks its required alignment";
    case W4A4_ERR_UNSUPPORTED: return "unsupported hadamard_block, or rank or K above the compiled maximum";
    case W4A4_ERR_HIP: return "HIP runtime error at launch";
    case W4A4_ERR_SCRATCH: return "the sizes need more workspace than the static buffer of svdq_linear_noalloc holds";
    default: return "unknown status";
  }
}

int w4a4_version(void) { return 100; }

w4a4_status svdq_quantize_act(const void* x, const void* smooth_factor, const void* proj_down, int64_t M, int64_t K,
                              int64_t R, int32_t hadamard_block, void* qact, void* ascales, float* lora_act,
                              void* stream) {
  w4a4_status st = validate_quantize_act(x, smooth_factor, proj_down, M, K, R, hadamard_block, qact, ascales, lora_act);
  if (st != W4A4_OK || M == 0) return st;
  (void)hipGetLastError();  // clear a stale error so it is not reported as ours
  return from_hip(w4a4::launch_quantize(true, x, smooth_factor, proj_down, M, K, R, hadamard_block, 1, qact, ascales,
                                        lora_act, static_cast<hipStream_t>(stream)));
}

w4a4_status svdq_quantize_weight(const void* w, const void* smooth_factor, int64_t N, int64_t K,
                                 int32_t hadamard_block, void* qweight, void* wscales, void* stream) {
  w4a4_status st = check_k_rank_block(K, 0, hadamard_block);
  if (st != W4A4_OK) return st;
  if (N < 0 || N > kMaxDim) return W4A4_ERR_SHAPE;
  if (N == 0) return W4A4_OK;
  if (!w || !smooth_factor || !qweight || !wscales) return W4A4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(smooth_factor, 16) || !aligned(qweight, 4)) return W4A4_ERR_ALIGN;
  (void)hipGetLastError();
  return from_hip(w4a4::launch_quantize(false, w, smooth_factor, nullptr, N, K, 0, hadamard_block, 1, qweight,
                                        wscales, nullptr, static_cast<hipStream_t>(stream)));
}

w4a4_status svdq_gemm_lowrank_bias(const void* qact, const void* ascales, const float* lora_act, const void* qweight,
                                   const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                                   const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                                   void* stream) {
  w4a4_status st = validate_gemm(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, M, N, K, R, y);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (bias && !aligned(bias, 2)) return W4A4_ERR_ALIGN;
  (void)hipGetLastError();
  return from_hip(w4a4::launch_gemm(qact, ascales, lora_act, 1, qweight, wscales, proj_up, wcscales, wtscale, bias, M,
                                    N, K, R, y, static_cast<hipStream_t>(stream)));
}

w4a4_status svdq_gemm_lowrank(const void* qact, const void* ascales, const float* lora_act, const void* qweight,
                              const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                              int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream) {
  return svdq_gemm_lowrank_bias(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, nullptr, M, N,
                                K, R, y, stream);
}

size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  if (M < 0 || M > kMaxDim || check_k_rank_block(K, R, 0) != W4A4_OK) return 0;
  const size_t m = (size_t)M, k = (size_t)K, r = (size_t)R;
  const size_t parts = (size_t)w4a4::quantize_parts(M, K);
  return align256(m * k / 2) + align256(k / 16 * m) + align256(parts * m * r * sizeof(float));
}

}  // extern "C"

namespace {

// svdq_linear's validation and, when `launch`, its two launches.  With launch == false nothing
// touches HIP and the workspace pointer is only checked (never dereferenced).
w4a4_status linear_impl(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                        const void* proj_up, const void* smooth_factor, const void* wcscales, const void* wtscale,
                        const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, int32_t hadamard_block, void* y,
                        void* workspace, size_t workspace_bytes, void* stream, bool launch) {
  w4a4_status st = check_k_rank_block(K, R, hadamard_block);
  if (st != W4A4_OK) return st;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return W4A4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !qweight || !wscales || !smooth_factor || !wcscales || !wtscale || !y) return W4A4_ERR_NULL;
  if (R > 0 && (!proj_down || !proj_up)) return W4A4_ERR_NULL;
  if (!workspace) return W4A4_ERR_NULL;
  const size_t need = svdq_linear_workspace_bytes(M, K, R);
  if (workspace_bytes < need) return W4A4_ERR_SHAPE;
  if (!aligned(workspace, 256) || (bias && !aligned(bias, 2))) return W4A4_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* qact = ws;
  void* ascales = ws + align256((size_t)M * K / 2);
  float* lora = R > 0 ? reinterpret_cast<float*>(ws + align256((size_t)M * K / 2) + align256((size_t)K / 16 * M))
                      : nullptr;
  st = validate_quantize_act(x, smooth_factor, proj_down, M, K, R, hadamard_block, qact, ascales, lora);
  if (st != W4A4_OK) return st;
  st = validate_gemm(qact, ascales, lora, qweight, wscales, proj_up, wcscales, wtscale, M, N, K, R, y);
  if (st != W4A4_OK || !launch) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int parts = w4a4::quantize_parts(M, K);
  st = from_hip(w4a4::launch_quantize(true, x, smooth_factor, proj_down, M, K, R, hadamard_block, parts, qact, ascales,
                                      lora, s));
  if (st != W4A4_OK) return st;
  return from_hip(w4a4::launch_gemm(qact, ascales, lora, parts, qweight, wscales, proj_up, wcscales, wtscale, bias, M,
                                    N, K, R, y, s));
}

}  // namespace

extern "C" {

w4a4_status svdq_linear_bias(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                             const void* proj_up, const void* smooth_factor, const void* wcscales,
                             const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                             int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(x, qweight, wscales, proj_down, proj_up, smooth_factor, wcscales, wtscale, bias, M, N, K, R,
                     hadamard_block, y, workspace, workspace_bytes, stream, true);
}

w4a4_status svdq_linear(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                        const void* proj_up, const void* smooth_factor, const void* wcscales, const void* wtscale,
                        int64_t M, int64_t N, int64_t K, int64_t R, int32_t hadamard_block, void* y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return svdq_linear_bias(x, qweight, wscales, proj_down, proj_up, smooth_factor, wcscales, wtscale, nullptr, M, N, K,
                          R, hadamard_block, y, workspace, workspace_bytes, stream);
}

w4a4_status svdq_linear_noalloc(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                                const void* proj_up, const void* smooth_factor, const void* wcscales,
                                const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                int32_t hadamard_block, void* y, void* stream) {
  // Every check of svdq_linear_bias first, with a stand-in address for the static buffer (it is
  // not dereferenced), so that invalid calls get the same status and touch no HIP state; then the
  // buffer's limit; then its address on the current device, and the same launches.
  const size_t cap = (size_t)W4A4_NOALLOC_SCRATCH_BYTES;
  void* const stand_in = reinterpret_cast<void*>(uintptr_t{256});
  w4a4_status st = linear_impl(x, qweight, wscales, proj_down, proj_up, smooth_factor, wcscales, wtscale, bias, M, N,
                               K, R, hadamard_block, y, stand_in, SIZE_MAX, stream, false);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (svdq_linear_workspace_bytes(M, K, R) > cap) return W4A4_ERR_SCRATCH;
  void* ws = w4a4::noalloc_scratch();
  if (ws == nullptr) return W4A4_ERR_HIP;
  return linear_impl(x, qweight, wscales, proj_down, proj_up, smooth_factor, wcscales, wtscale, bias, M, N, K, R,
                     hadamard_block, y, ws, cap, stream, true);
}

}  // extern "C"

// ---- MXFP4 variant -----------------------------------------------------------------------

namespace {

int64_t mx_rows(int64_t M) { return (M + 3) / 4 * 4; }

w4a4_status check_mx(int64_t K, int64_t R, int32_t hb, bool gemm) {
  if (hb != 0 && hb != 32) return W4A4_ERR_UNSUPPORTED;
  w4a4_status st = check_k_rank_block(K, R, hb);
  if (st != W4A4_OK) return st;
  if (K % (gemm ? 128 : 32) != 0) return W4A4_ERR_SHAPE;
  return W4A4_OK;
}

w4a4_status validate_gemm_mx(const void* qact, const void* ascales, const float* lora, const void* qweight,
                             const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                             int64_t M, int64_t N, int64_t K, int64_t R, const void* y) {
  w4a4_status st = check_mx(K, R, 0, true);
  if (st != W4A4_OK) return st;
  if (N % 4 != 0) return W4A4_ERR_SHAPE;
  st = validate_gemm(qact, ascales, lora, qweight, wscales, proj_up, wcscales, wtscale, M, N, K, R, y);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (!aligned(ascales, 4) || !aligned(wscales, 4)) return W4A4_ERR_ALIGN;
  return W4A4_OK;
}

}  // namespace

extern "C" {

w4a4_status svdq_quantize_act_mx(const void* x, const void* smooth_factor, const void* proj_down, int64_t M,
                                 int64_t K, int64_t R, int32_t hadamard_block, void* qact, void* ascales,
                                 float* lora_act, void* stream) {
  w4a4_status st = check_mx(K, R, hadamard_block, false);
  if (st != W4A4_OK) return st;
  st = validate_quantize_act(x, smooth_factor, proj_down, M, K, R, hadamard_block, qact, ascales, lora_act);
  if (st != W4A4_OK || M == 0) return st;
  (void)hipGetLastError();
  return from_hip(w4a4::launch_quantize(true, x, smooth_factor, proj_down, M, K, R, hadamard_block, 1, qact, ascales,
                                        lora_act, static_cast<hipStream_t>(stream), true, mx_rows(M)));
}

w4a4_status svdq_quantize_weight_mx(const void* w, const void* smooth_factor, int64_t N, int64_t K,
                                    int32_t hadamard_block, void* qweight, void* wscales, void* stream) {
  w4a4_status st = check_mx(K, 0, hadamard_block, false);
  if (st != W4A4_OK) return st;
  if (N < 0 || N > kMaxDim) return W4A4_ERR_SHAPE;
  if (N == 0) return W4A4_OK;
  if (!w || !smooth_factor || !qweight || !wscales) return W4A4_ERR_NULL;
  if (!aligned(w, 16) || !aligned(smooth_factor, 16) || !aligned(qweight, 4)) return W4A4_ERR_ALIGN;
  (void)hipGetLastError();
  return from_hip(w4a4::launch_quantize(false, w, smooth_factor, nullptr, N, K, 0, hadamard_block, 1, qweight,
                                        wscales, nullptr, static_cast<hipStream_t>(stream), true, N));
}

w4a4_status svdq_gemm_lowrank_mx_bias(const void* qact, const void* ascales, const float* lora_act,
                                      const void* qweight, const void* wscales, const void* proj_up,
                                      const void* wcscales, const void* wtscale, const void* bias, int64_t M,
                                      int64_t N, int64_t K, int64_t R, void* y, void* stream) {
  w4a4_status st =
      validate_gemm_mx(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, M, N, K, R, y);
  if (st != W4A4_OK || M == 0 || N == 0) return st;
  if (bias && !aligned(bias, 2)) return W4A4_ERR_ALIGN;
  (void)hipGetLastError();
  return from_hip(w4a4::launch_gemm_mx(qact, ascales, lora_act, 1, qweight, wscales, proj_up, wcscales, wtscale, bias,
                                       M, N, K, R, mx_rows(M), y, static_cast<hipStream_t>(stream)));
}

w4a4_status svdq_gemm_lowrank_mx(const void* qact, const void* ascales, const float* lora_act, const void* qweight,
                                 const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                                 int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream) {
  return svdq_gemm_lowrank_mx_bias(qact, ascales, lora_act, qweight, wscales, proj_up, wcscales, wtscale, nullptr, M,
                                   N, K, R, y, stream);
}

size_t svdq_linear_mx_workspace_bytes(int64_t M, int64_t K, int64_t R) {
  if (M < 0 || M > kMaxDim || check_mx(K, R, 0, false) != W4A4_OK) return 0;
  const size_t m = (size_t)M, k = (size_t)K, r = (size_t)R;
  const size_t parts = (size_t)w4a4::quantize_parts(M, K);
  return align256(m * k / 2) + align256(k / 32 * (size_t)mx_rows(M)) + align256(parts * m * r * sizeof(float));
}

w4a4_status svdq_linear_mx_bias(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                                const void* proj_up, const void* smooth_factor, const void* wcscales,
                                const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes,
                                void* stream) {
  w4a4_status st = check_mx(K, R, hadamard_block, true);
  if (st != W4A4_OK) return st;
  if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim || N % 4 != 0) return W4A4_ERR_SHAPE;
  if (M == 0 || N == 0) return W4A4_OK;
  if (!x || !qweight || !wscales || !smooth_factor || !wcscales || !wtscale || !y) return W4A4_ERR_NULL;
  if (R > 0 && (!proj_down || !proj_up)) return W4A4_ERR_NULL;
  if (!workspace) return W4A4_ERR_NULL;
  const size_t need = svdq_linear_mx_workspace_bytes(M, K, R);
  if (workspace_bytes < need) return W4A4_ERR_SHAPE;
  if (!aligned(workspace, 256) || (bias && !aligned(bias, 2))) return W4A4_ERR_ALIGN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* qact = ws;
  void* ascales = ws + align256((size_t)M * K / 2);
  float* lora = R > 0 ? reinterpret_cast<float*>(ws + align256((size_t)M * K / 2) +
                                                 align256((size_t)K / 32 * (size_t)mx_rows(M)))
                      : nullptr;
  st = validate_quantize_act(x, smooth_factor, proj_down, M, K, R, hadamard_block, qact, ascales, lora);
  if (st != W4A4_OK) return st;
  st = validate_gemm_mx(qact, ascales, lora, qweight, wscales, proj_up, wcscales, wtscale, M, N, K, R, y);
  if (st != W4A4_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int parts = w4a4::quantize_parts(M, K);
  st = from_hip(w4a4::launch_quantize(true, x, smooth_factor, proj_down, M, K, R, hadamard_block, parts, qact, ascales,
                                      lora, s, true, mx_rows(M)));
  if (st != W4A4_OK) return st;
  return from_hip(w4a4::launch_gemm_mx(qact, ascales, lora, parts, qweight, wscales, proj_up, wcscales, wtscale, bias,
                                       M, N, K, R, mx_rows(M), y, s));
}

w4a4_status svdq_linear_mx(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                           const void* proj_up, const void* smooth_factor, const void* wcscales, const void* wtscale,
                           int64_t M, int64_t N, int64_t K, int64_t R, int32_t hadamard_block, void* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return svdq_linear_mx_bias(x, qweight, wscales, proj_down, proj_up, smooth_factor, wcscales, wtscale, nullptr, M, N,
                             K, R, hadamard_block, y, workspace, workspace_bytes, stream);
}

// ---- standalone block Hadamard transform (rotate notes, section 3.1) ------------------------

w4a4_status w4a4_hadamard_transform(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                                    int32_t block, int32_t dtype, void* stream) {
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > (int64_t)1 << 30) return W4A4_ERR_SHAPE;
  if (block < 2 || block > W4A4_HADAMARD_MAX_BLOCK || (block & (block - 1)) != 0) return W4A4_ERR_UNSUPPORTED;
  if (dtype < W4A4_DTYPE_BF16 || dtype > W4A4_DTYPE_F32) return W4A4_ERR_UNSUPPORTED;
  if (cols % block != 0 || ldx < cols || ldy < cols) return W4A4_ERR_SHAPE;
  if (x == y && ldx != ldy) return W4A4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return W4A4_OK;
  if (!x || !y) return W4A4_ERR_NULL;
  const uintptr_t es = dtype == W4A4_DTYPE_F32 ? 4 : 2;
  if (!aligned(x, es) || !aligned(y, es)) return W4A4_ERR_ALIGN;
  const float norm = (float)(1.0 / std::sqrt((double)block));
  (void)hipGetLastError();
  return from_hip(
      w4a4::launch_hadamard(x, ldx, y, ldy, rows, cols, block, dtype, norm, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
