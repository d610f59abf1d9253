/*
 * libw4a4 -- SVDQuant W4A4 quantized linear layer for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Every tensor argument is a device pointer on the current HIP
 * device, dense and row-major in the shape given; the caller owns every
 * buffer.  All work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL is the default stream).  No entry point allocates, frees or
 * synchronizes.  Validation happens before any launch: a call that returns an
 * error has launched nothing and written nothing.  Faults during execution
 * surface at the caller's next synchronization.  Calls are thread-safe (for
 * svdq_linear_noalloc see its note on overlapping calls); no call depends on an
 * earlier one.  The library caches, once per device and atomically, the CU count,
 * the occupancy of its persistent kernels and the address of the static buffer
 * of svdq_linear_noalloc.  Checks run in this order: sizes
 * (W4A4_ERR_SHAPE / W4A4_ERR_UNSUPPORTED), the empty call (M or N == 0 is
 * valid, launches nothing and may pass NULL pointers), NULL pointers
 * (W4A4_ERR_NULL), alignment (W4A4_ERR_ALIGN).
 *
 * Formats (from the "SVDQuant W4A4" page, section "Checkpoint contract",
 * configuration precision "nvfp4"):
 *   FP4      E2M1, two values per byte, the even-k element in the low nibble;
 *   scales   float8_e4m3fn bytes, one per 16 consecutive inputs along K;
 *   bf16     IEEE bfloat16.
 *
 * Method (same page, sections "Overview" and "Runtime support"; rotation from
 * the rotate notes, sections 2.1-2.2 and 3.3): y = x W^T is computed as
 *   x_s   = x / smooth_factor                            (float32, IEEE)
 *   v     = x_s @ H_B^T per B-block of K                 (optional rotation)
 *   qact, ascales = per-16 group FP4 quantization of v   (amax/6 -> e4m3)
 *   y     = bf16( (dequant(qact) @ dequant(qweight)^T) * wcscales * wtscale
 *                 + (x_s @ proj_down) @ proj_up^T )
 * with the weight-side smoothing and rotation folded into qweight offline.
 */
#ifndef W4A4_H_
#define W4A4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_NULL = 1,        /* a required pointer is NULL                         */
  W4A4_ERR_SHAPE = 2,       /* a size is negative, K % 16 != 0, K % block != 0,
                               or the workspace is too small                      */
  W4A4_ERR_ALIGN = 3,       /* a pointer breaks its required alignment            */
  W4A4_ERR_UNSUPPORTED = 4, /* hadamard_block not in {0,16,32,64,128}, R > 64, or K > W4A4_MAX_K */
  W4A4_ERR_HIP = 5,         /* the HIP runtime reported an error at launch        */
  W4A4_ERR_SCRATCH = 6      /* svdq_linear_noalloc: the sizes need more workspace than its static
                               device buffer holds (W4A4_NOALLOC_SCRATCH_BYTES)   */
} w4a4_status;

/* Largest supported correction rank R. */
#define W4A4_MAX_RANK 64
/* Largest supported K (2^24 columns): the kernels address a tile's rows x K/2 code bytes with
   32-bit offsets. */
#define W4A4_MAX_K (1 << 24)

/* Human-readable name of a status code (static storage). */
const char* w4a4_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int w4a4_version(void);

/*
 * Online activation quantizer ("SVDQuant W4A4" page, "Runtime support": BF16
 * input; rotation: rotate notes 2.1 and 3.3, quantization fused with the
 * rotation in one pass).  One HBM pass over x computes, per row m:
 *   x_s  = float32(x) / float32(smooth_factor)                  (IEEE division)
 *   v    = x_s, or x_s @ H_B^T on every contiguous B-block when hadamard_block
 *          B > 0 (Sylvester order, butterfly spans 1,2,...,B/2, then one
 *          multiply by float32(1/sqrt(B)))
 *   per group g of 16:  s8 = e4m3(amax|v| / 6)  (round-nearest-even, saturating
 *          at 448);  code = e2m1(v / e4m3_value(s8))  (round-nearest-even,
 *          saturating at 6, sign of zero kept), all codes 0 when s8 == 0
 *   lora_act = x_s @ proj_down       (unrotated x_s, float32 result)
 *
 *   x             bf16 [M, K]           16-byte aligned
 *   smooth_factor bf16 [K]
 *   proj_down     bf16 [K, R]           may be NULL when R == 0
 *   M >= 0, K >= 16 with K % 16 == 0, 0 <= R <= 64
 *   hadamard_block  0 (none) or 16, 32, 64, 128 with K % hadamard_block == 0
 *   qact          u8   [M, K/2]  out    E2M1 pairs, 4-byte aligned
 *   ascales       u8   [K/16, M] out    e4m3 bytes (layout mirrors wscales)
 *   lora_act      f32  [M, R]    out    may be NULL when R == 0
 * M == 0 is a valid empty call (nothing is launched).
 */
w4a4_status svdq_quantize_act(const void* x, const void* smooth_factor, const void* proj_down,
                              int64_t M, int64_t K, int64_t R, int32_t hadamard_block,
                              void* qact, void* ascales, float* lora_act, void* stream);

/*
 * Offline weight quantizer producing the checkpoint tensors ("SVDQuant W4A4"
 * page, "Checkpoint contract": qweight (N, K/2) packed FP4, wscales (K/16, N)
 * e4m3; rotate notes 2.1: weights are rotated offline, W' = R W).  Per row n:
 *   w_s = float32(w) * float32(smooth_factor)    (exact for bf16 inputs)
 *   v   = w_s, or w_s @ H_B^T per B-block (as in svdq_quantize_act)
 *   per-16 group quantization exactly as in svdq_quantize_act.
 *
 *   w        bf16 [N, K]   16-byte aligned
 *   smooth_factor bf16 [K]
 *   qweight  u8   [N, K/2] out   4-byte aligned
 *   wscales  u8   [K/16, N] out
 */
w4a4_status svdq_quantize_weight(const void* w, const void* smooth_factor, int64_t N, int64_t K,
                                 int32_t hadamard_block, void* qweight, void* wscales, void* stream);

/*
 * Block-scaled FP4 GEMM with the low-rank correction fused in the epilogue
 * ("SVDQuant W4A4" page, "Runtime support": NVFP4 GEMM followed by the BF16
 * rank correction; "Checkpoint contract": proj_up, wcscales, wtscale):
 *   y[m,n] = bf16( sum_k e2m1(qact[m,k]) e4m3(ascales[k/16,m])
 *                        e2m1(qweight[n,k]) e4m3(wscales[k/16,n])
 *                  * wcscales[n] * wtscale
 *                  + sum_r lora_act[m,r] proj_up[n,r] )
 * The products are exact; the sum is accumulated in float32 (matrix cores).
 *
 *   qact     u8   [M, K/2]   16-byte aligned     ascales u8 [K/16, M]
 *   lora_act f32  [M, R]     may be NULL when R == 0
 *   qweight  u8   [N, K/2]   16-byte aligned     wscales u8 [K/16, N]
 *   proj_up  bf16 [N, R]     may be NULL when R == 0
 *   wcscales bf16 [N]
 *   wtscale  bf16 [1]        device scalar, read by the kernel
 *   y        bf16 [M, N] out
 */
w4a4_status svdq_gemm_lowrank(const void* qact, const void* ascales, const float* lora_act,
                              const void* qweight, const void* wscales, const void* proj_up,
                              const void* wcscales, const void* wtscale,
                              int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream);

/* Bytes of workspace svdq_linear needs for these sizes (qact, ascales and
 * lora_act, each 256-byte aligned).  Returns 0 for invalid sizes. */
size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int64_t R);

/*
 * The whole layer: svdq_quantize_act into the workspace, then
 * svdq_gemm_lowrank.  Arguments are the checkpoint tensors of the "SVDQuant
 * W4A4" page's table plus the BF16 input x [M, K] and the output y [M, N].
 * `workspace` is device memory of at least svdq_linear_workspace_bytes(M, K, R)
 * bytes, 256-byte aligned; its contents need no initialisation and are
 * overwritten.
 */
w4a4_status svdq_linear(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                        const void* proj_up, const void* smooth_factor, const void* wcscales,
                        const void* wtscale, int64_t M, int64_t N, int64_t K, int64_t R,
                        int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes,
                        void* stream);


/*
 * MXFP4 variant of the layer (rotate notes, section 3.3, FP-Quant:
 * hadamard_group_size 32, forward_dtype "mxfp4", forward_method "abs_max";
 * fused_quantize_mx then matmul_mxf4_bf16).  Smoothing, the optional rotation
 * and the low-rank branch are those of the entry points above; the
 * quantization works on blocks of 32 consecutive K-columns with one E8M0
 * (power-of-two) scale per block instead of 16-groups with e4m3 scales:
 *   e     = the least integer with 2^e >= f32(amax|v| / 6), clamped to [-127, 127]
 *   scale byte = e + 127  (E8M0: value 2^(byte - 127))
 *   code  = e2m1(v * 2^-e)   (round-to-nearest-even, saturating at 6, sign kept)
 * and the GEMM multiplies E2M1 codes scaled by 2^(byte - 127) per row and block
 * (matrix-core instruction with per-block power-of-two scales), fp32
 * accumulation, the same epilogue.  Inputs must be finite.
 *
 * svdq_quantize_act_mx: as svdq_quantize_act with K % 32 == 0 and
 *   hadamard_block 0 or 32;
 *   ascales  u8 [K/32, Mp] out   Mp = 4 * ceil(M / 4); columns M .. Mp-1 are written 0
 * svdq_quantize_weight_mx: as svdq_quantize_weight with K % 32 == 0 and
 *   hadamard_block 0 or 32;  wscales u8 [K/32, N] out
 * svdq_gemm_lowrank_mx: as svdq_gemm_lowrank with K % 128 == 0, N % 4 == 0;
 *   ascales u8 [K/32, Mp] and wscales u8 [K/32, N], both 4-byte aligned
 * svdq_linear_mx: svdq_quantize_act_mx into the workspace (at least
 *   svdq_linear_mx_workspace_bytes(M, K, R) bytes, 256-byte aligned), then
 *   svdq_gemm_lowrank_mx.
 * Other sizes return W4A4_ERR_SHAPE (K, N) or W4A4_ERR_UNSUPPORTED (hadamard_block).
 */
w4a4_status svdq_quantize_act_mx(const void* x, const void* smooth_factor, const void* proj_down,
                                 int64_t M, int64_t K, int64_t R, int32_t hadamard_block,
                                 void* qact, void* ascales, float* lora_act, void* stream);

w4a4_status svdq_quantize_weight_mx(const void* w, const void* smooth_factor, int64_t N, int64_t K,
                                    int32_t hadamard_block, void* qweight, void* wscales, void* stream);

w4a4_status svdq_gemm_lowrank_mx(const void* qact, const void* ascales, const float* lora_act,
                                 const void* qweight, const void* wscales, const void* proj_up,
                                 const void* wcscales, const void* wtscale,
                                 int64_t M, int64_t N, int64_t K, int64_t R, void* y, void* stream);

size_t svdq_linear_mx_workspace_bytes(int64_t M, int64_t K, int64_t R);

w4a4_status svdq_linear_mx(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                           const void* proj_up, const void* smooth_factor, const void* wcscales,
                           const void* wtscale, int64_t M, int64_t N, int64_t K, int64_t R,
                           int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ---- Optional bias -------------------------------------------------------------------------
 * Rotate notes, section 3.2: the linear-layer wrapper hands the layer's optional bias to the
 * quantized method (apply(layer, x, bias)).  These four entry points are the ones above with one
 * more argument, `bias`: bf16 [N] (2-byte aligned) or NULL for none.  It is added in float32 to
 * each output after the scaled quantized product and the low-rank term, before the single
 * rounding to bf16, and is not multiplied by wcscales or wtscale:
 *   y = bf16( acc * wcscales * wtscale + L @ proj_up^T + bias )
 * Validation and errors are those of the entry point without bias, plus W4A4_ERR_ALIGN for an
 * odd bias address. */
w4a4_status svdq_gemm_lowrank_bias(const void* qact, const void* ascales, const float* lora_act,
                                   const void* qweight, const void* wscales, const void* proj_up,
                                   const void* wcscales, const void* wtscale, const void* bias, int64_t M,
                                   int64_t N, int64_t K, int64_t R, void* y, void* stream);
w4a4_status svdq_linear_bias(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                             const void* proj_up, const void* smooth_factor, const void* wcscales,
                             const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                             int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes,
                             void* stream);
w4a4_status svdq_gemm_lowrank_mx_bias(const void* qact, const void* ascales, const float* lora_act,
                                      const void* qweight, const void* wscales, const void* proj_up,
                                      const void* wcscales, const void* wtscale, const void* bias, int64_t M,
                                      int64_t N, int64_t K, int64_t R, void* y, void* stream);
w4a4_status svdq_linear_mx_bias(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                                const void* proj_up, const void* smooth_factor, const void* wcscales,
                                const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                int32_t hadamard_block, void* y, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- The layer without allocation ---------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  svdq_linear_bias (bias may be NULL) with its workspace
 * in a static device buffer of W4A4_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU
 * it runs on until the process ends, instead of a caller-provided one.  Same kernels, same
 * results bit for bit.  Calls whose workspace (svdq_linear_workspace_bytes(M, K, R)) exceeds the
 * buffer return W4A4_ERR_SCRATCH before any HIP call; other errors as for svdq_linear_bias.  The
 * call allocates and frees nothing; the buffer's address is looked up once per device (on the
 * first call with that device current).  Every call on one GPU uses that GPU's one buffer, so
 * calls that may overlap on a GPU (concurrent streams, host threads) race and must be ordered by
 * the caller. */
#define W4A4_NOALLOC_SCRATCH_BYTES (64u << 20)
w4a4_status svdq_linear_noalloc(const void* x, const void* qweight, const void* wscales, const void* proj_down,
                                const void* proj_up, const void* smooth_factor, const void* wcscales,
                                const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                int32_t hadamard_block, void* y, void* stream);

/* ---- Offline low-rank split (host) ----------------------------------------------------------
 * "SVDQuant W4A4" page, "Overview" (four-bit weights and activations plus a small low-rank
 * branch that corrects part of the quantization error; checkpoints are quantized offline) and
 * "Checkpoint contract" (proj_down (K, R), proj_up (N, R)).  HOST memory throughout; no GPU
 * work.  With W_s = W * smooth_factor (float64) and its top-R singular triplets U_R S_R V_R:
 *   proj_up   = bf16(U_R sqrt(S_R))         [N, R] bf16
 *   proj_down = bf16(V_R sqrt(S_R))         [K, R] bf16
 *   residual  = bf16(W_s - proj_up proj_down^T)   [N, K] bf16 (smoothing already applied: quantize
 *               it with svdq_quantize_weight and a smooth_factor of ones to get qweight, wscales)
 *   singular_values  S_1 >= ... >= S_R as float (may be NULL)
 * The triplets come from a randomized range finder with R + oversample Gaussian columns (drawn
 * from `seed`) and `power_iters` power iterations; `threads` host threads (<= 0: all cores).
 * Sizes: 1 <= N, K <= 2^20, N * K <= 2^31, 0 <= R <= min(N, K, W4A4_MAX_RANK), oversample >= 0,
 * power_iters >= 0, else W4A4_ERR_SHAPE; NULL w, smooth_factor or residual (or factors with
 * R > 0): W4A4_ERR_NULL.  R == 0 writes the smoothed weight to residual. */
w4a4_status svdq_lowrank_split(const void* w, const void* smooth_factor, int64_t N, int64_t K, int64_t R,
                               int32_t oversample, int32_t power_iters, uint64_t seed, int32_t threads,
                               void* proj_down, void* proj_up, void* residual, float* singular_values);

/* ---- Standalone block Hadamard transform ------------------------------------------------
 * Rotate notes, section 3.1 (the Hadacore kernel behind hadacore_transform(x, inplace): the
 * Sylvester Hadamard transform applied through its recursion, symmetric and therefore its own
 * inverse, in place or not) and section 3.2 (applied per head_dim block, and to column
 * partitions [start, start + length) of a layer's output); the Sylvester recursion and the
 * 1/sqrt(n) normalisation from sections 2.1-2.2.
 *
 * For each of `rows` rows and each block of `block` consecutive columns of the first `cols`:
 *   y[r, blk] = round( float32(1/sqrt(block)) * FWHT(float32(x[r, blk])) )
 * with butterfly spans 1, 2, ..., block/2 in that order, each pair (a, b) -> (a + b, a - b) in
 * float32, one multiply, then one round to nearest even into the storage type (bf16 and f16;
 * f32 is stored as computed).  Results are bit-identical to that sequence of float32
 * operations (the quantizers' fused rotation uses the same one).
 *   x, y   device pointers to element (0, 0); row r starts ldx (ldy) elements after row r - 1,
 *          so a column partition is addressed as x + start with the full row stride.
 *   ldx, ldy  row strides in elements, >= cols.
 *   dtype  W4A4_DTYPE_BF16, W4A4_DTYPE_F16 or W4A4_DTYPE_F32 (both tensors).
 *   block  a power of two in [2, W4A4_HADAMARD_MAX_BLOCK]; cols % block == 0.
 * x == y (with ldx == ldy) transforms in place; any other overlap of x and y is undefined.
 * Columns at and past `cols` in each row are not touched.  Errors: W4A4_ERR_SHAPE (negative
 * sizes, cols % block, ld < cols, x == y with ldx != ldy), W4A4_ERR_UNSUPPORTED (block,
 * dtype), W4A4_ERR_NULL, W4A4_ERR_ALIGN (x or y not aligned to the element size).  rows == 0
 * or cols == 0 launches nothing.  16-byte aligned pointers, row strides and column counts that
 * are multiples of 8 take the vectorised path. */
#define W4A4_DTYPE_BF16 0
#define W4A4_DTYPE_F16 1
#define W4A4_DTYPE_F32 2
#define W4A4_HADAMARD_MAX_BLOCK 4096
w4a4_status w4a4_hadamard_transform(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                                    int32_t block, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H_ */
