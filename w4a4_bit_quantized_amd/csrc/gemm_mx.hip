// MXFP4 variant of the block-scaled GEMM (gfx950), with the low-rank epilogue of gemm.hip
// (rotate notes, section 3.3: FP-Quant mxfp4, matmul_mxf4_bf16).
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

// ---- MXFP4 variant (rotate notes, section 3.3: FP-Quant mxfp4, matmul_mxf4_bf16) ----------
// Codes as above; one E8M0 scale per 32 K-columns, (K/32, rows) tensors whose dwords are 4
// consecutive rows of one block.  The product runs on the scaled FP4 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4, which takes the packed E2M1 codes directly and applies a
// power-of-two scale per row and 32-column block: no decode.  Lane l of an operand supplies row
// l % 32, K-columns 32 (l / 32) .. +32 of the instruction's 64 (16 bytes in the first four
// registers) and, in byte `opsel` of its scale register, the E8M0 byte of that row and block.
// A K-step of 128 columns is two instructions; lane half h reads code chunks h and 2 + h of
// its row and the scales of blocks h and 2 + h.  The accumulator layout equals the f16
// kernel's, so the epilogue is shared.
template <class T, int S>
struct DmaTileMx {
  static constexpr int STAGES = S;                // K-steps resident in LDS; S - 1 of them in flight
  static constexpr int WAVES = T::WM * T::WN;
  static constexpr int ROUND_ROWS = 16 * WAVES;
  static constexpr int ROUNDS = (T::ROWS + ROUND_ROWS - 1) / ROUND_ROWS;
  static constexpr int SDW = T::ROWS;             // scale dwords per K-step: ROWS/4 quads x 4 blocks
  static constexpr int SROUNDS = (SDW + 64 * WAVES - 1) / (64 * WAVES);
  static constexpr int SCALE_OFF = ROUNDS * ROUND_ROWS * 64;
  static constexpr int STAGE = SCALE_OFF + SROUNDS * WAVES * 256;
  static constexpr int LOADS = ROUNDS + SROUNDS;
  static constexpr int LDS_BYTES = S * STAGE > T::EPI_LDS ? S * STAGE : T::EPI_LDS;
  static_assert(T::BM % 16 == 0 && T::ROWS % 16 == 0, "whole 16-row blocks");
  static_assert(S >= 3 && (S - 2) * LOADS < 64, "vmcnt range");
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Read a wave's operands of one K-step from its LDS stage, the scale dwords as read (two per
// fragment: blocks h and 2 + h), combined only where they are used.  Fragment and wave row offsets
// are multiples of 32, so a row's chunk swizzle depends on l32 alone: every read is a per-lane base
// plus an immediate.
template <class T, class D>
__device__ __forceinline__ void mx_read_raw(const uint8_t* cur, int wm, int wn, int l32, int h,
                                            uint32_t (&qA)[T::FRAG_M][2], uint32_t (&qB)[T::FRAG_N][2],
                                            i32x4_t (&cA)[2][T::FRAG_M], i32x4_t (&cB)[2][T::FRAG_N]) {
  const int sw4 = (l32 >> 2) & 3;
  const int ra = wm * T::FRAG_M * 32 + l32, rb = T::BM + wn * T::FRAG_N * 32 + l32;
#pragma unroll
  for (int i = 0; i < T::FRAG_M; ++i) {
    const uint32_t* sq = reinterpret_cast<const uint32_t*>(cur + D::SCALE_OFF + (ra >> 2) * 16 + i * 8 * 16);
    qA[i][0] = sq[h];
    qA[i][1] = sq[2 + h];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      cA[s2][i] = *reinterpret_cast<const i32x4_t*>(cur + ra * 64 + 16 * ((2 * s2 + h) ^ sw4) + i * 32 * 64);
  }
#pragma unroll
  for (int j = 0; j < T::FRAG_N; ++j) {
    const uint32_t* sq = reinterpret_cast<const uint32_t*>(cur + D::SCALE_OFF + (rb >> 2) * 16 + j * 8 * 16);
    qB[j][0] = sq[h];
    qB[j][1] = sq[2 + h];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      cB[s2][j] = *reinterpret_cast<const i32x4_t*>(cur + rb * 64 + 16 * ((2 * s2 + h) ^ sw4) + j * 32 * 64);
  }
}

// One K-step on the matrix cores: weights first (output columns n), activations second (output
// rows m), as in the f16 kernel.
template <int FM, int FN>
__device__ __forceinline__ void mx_mma(float16_t (&acc)[FM][FN], const uint32_t (&sA)[FM], const uint32_t (&sB)[FN],
                                       const i32x4_t (&cA)[2][FM], const i32x4_t (&cB)[2][FN]) {
  // FP4 operands occupy the first four registers of the instruction's eight
  auto w = [](i32x4_t c) { return __builtin_shufflevector(c, c, 0, 1, 2, 3, -1, -1, -1, -1); };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w(cB[0][j]), w(cA[0][i]), acc[i][j], 4, 4, 0, sB[j], 0,
                                                                  sA[i]);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w(cB[1][j]), w(cA[1][i]), acc[i][j], 4, 4, 1, sB[j], 1,
                                                                  sA[i]);
}

// Half-step pieces of the interleaved loop: the code chunks of instruction s2 of every fragment, the
// raw scale dwords (blocks h and 2 + h) of every fragment, and the matrix instructions of one half.
template <class T, class D>
__device__ __forceinline__ void mx_read_codes(const uint8_t* cur, int wm, int wn, int l32, int h, int s2,
                                              i32x4_t (&cA)[T::FRAG_M], i32x4_t (&cB)[T::FRAG_N]) {
  const int sw4 = (l32 >> 2) & 3;
  const int ra = wm * T::FRAG_M * 32 + l32, rb = T::BM + wn * T::FRAG_N * 32 + l32;
#pragma unroll
  for (int i = 0; i < T::FRAG_M; ++i)
    cA[i] = *reinterpret_cast<const i32x4_t*>(cur + ra * 64 + 16 * ((2 * s2 + h) ^ sw4) + i * 32 * 64);
#pragma unroll
  for (int j = 0; j < T::FRAG_N; ++j)
    cB[j] = *reinterpret_cast<const i32x4_t*>(cur + rb * 64 + 16 * ((2 * s2 + h) ^ sw4) + j * 32 * 64);
}

template <class T, class D>
__device__ __forceinline__ void mx_read_scales(const uint8_t* cur, int wm, int wn, int l32, int h,
                                               uint32_t (&qA)[T::FRAG_M][2], uint32_t (&qB)[T::FRAG_N][2]) {
  const int ra = wm * T::FRAG_M * 32 + l32, rb = T::BM + wn * T::FRAG_N * 32 + l32;
#pragma unroll
  for (int i = 0; i < T::FRAG_M; ++i) {
    const uint32_t* sq = reinterpret_cast<const uint32_t*>(cur + D::SCALE_OFF + (ra >> 2) * 16 + i * 8 * 16);
    qA[i][0] = sq[h];
    qA[i][1] = sq[2 + h];
  }
#pragma unroll
  for (int j = 0; j < T::FRAG_N; ++j) {
    const uint32_t* sq = reinterpret_cast<const uint32_t*>(cur + D::SCALE_OFF + (rb >> 2) * 16 + j * 8 * 16);
    qB[j][0] = sq[h];
    qB[j][1] = sq[2 + h];
  }
}

template <int FM, int FN, int S2>
__device__ __forceinline__ void mx_mma_half(float16_t (&acc)[FM][FN], const uint32_t (&sA)[FM],
                                            const uint32_t (&sB)[FN], const i32x4_t (&cA)[FM],
                                            const i32x4_t (&cB)[FN]) {
  auto w = [](i32x4_t c) { return __builtin_shufflevector(c, c, 0, 1, 2, 3, -1, -1, -1, -1); };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w(cB[j]), w(cA[i]), acc[i][j], 4, 4, S2, sB[j], S2,
                                                                  sA[i]);
}

// K-step kt of the register-prefetching loop: operands of kt are in (qA, qB, cA, cB); those of
// kt + 1 are read into (nA, nB, dA, dB) while kt multiplies.  Once every wave holds K-step kt in
// registers, its slot `sl` = kt % S is refilled with K-step kt + S.  Past the last K-step the
// last one is reloaded and re-read, so every step issues the same loads (uniform vmcnt) and
// runs without branches.  The matrix instructions are interleaved with the LDS reads and the
// direct loads (one wave per SIMD: nothing else fills the matrix pipe while this wave stalls).
template <class T, class D, int S>
__device__ __forceinline__ void mx_pf_step(int kt, int sl, int nkt, uint8_t* lds,
                                           float16_t (&acc)[T::FRAG_M][T::FRAG_N], int wave, int wm, int wn, int l32,
                                           int h, uint32_t psel, const uint8_t* const* c_base, const uint32_t* c_off,
                                           const uint8_t* const* s_base, const uint32_t* s_off,
                                           const uint32_t* s_stride, const uint32_t (&qA)[T::FRAG_M][2],
                                           const uint32_t (&qB)[T::FRAG_N][2], const i32x4_t (&cA)[2][T::FRAG_M],
                                           const i32x4_t (&cB)[2][T::FRAG_N], uint32_t (&nA)[T::FRAG_M][2],
                                           uint32_t (&nB)[T::FRAG_N][2], i32x4_t (&dA)[2][T::FRAG_M],
                                           i32x4_t (&dB)[2][T::FRAG_N]) {
  constexpr int FM = T::FRAG_M, FN = T::FRAG_N;
  vm_wait_barrier<(S - 2) * D::LOADS>();  // K-step kt + 1 has landed
  uint32_t sA[FM], sB[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) sA[i] = __builtin_amdgcn_perm(qA[i][1], qA[i][0], psel);
#pragma unroll
  for (int j = 0; j < FN; ++j) sB[j] = __builtin_amdgcn_perm(qB[j][1], qB[j][0], psel);
  const int kn = min(kt + S, nkt - 1);
  dma_issue<D>(lds + sl * D::STAGE, wave, (uint32_t)kn * (BK / 2), (size_t)kn * (BK / 32), c_base, c_off, s_base,
               s_off, s_stride);
  const int sn = sl == S - 1 ? 0 : sl + 1;
  mx_read_raw<T, D>(lds + sn * D::STAGE, wm, wn, l32, h, nA, nB, dA, dB);
  mx_mma(acc, sA, sB, cA, cB);
  // per matrix instruction of the first 2 (FM + FN): two LDS reads and one direct load
#pragma unroll
  for (int g = 0; g < 2 * (FM + FN); ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // vector memory read
  }
}

// `ms` is the row stride of the activation scale tensor (M rounded up to 4).  PF selects the
// register-prefetching K loop (for one wave per SIMD, whose LDS latency no other wave hides).
template <int WAVES_M, int WAVES_N, int FM, int FN, int S, bool PF, bool LORA>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_mx_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R, int ms,
    uint16_t* __restrict__ y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  using D = DmaTileMx<T, S>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[D::LDS_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform: wave-level addresses in scalar registers
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  int tm, tn;
  tile_of((int)blockIdx.x, (int)gridDim.x, (M + T::BM - 1) / T::BM, tiles_n, tm, tn);
  const int n0 = tn * T::BN;
  const int m0 = tm * T::BM;
  const uint32_t kbytes = (uint32_t)K / 2;
  const int nkt = K / BK;
  const int rows_a = min(T::BM, M - m0), rows_b = min(T::BN, N - n0);
  const int srows_a = min(T::BM, ms - m0);  // scale rows: whole quads (ms % 4 == 0, N % 4 == 0)

  const uint8_t* c_base[D::ROUNDS];
  uint32_t c_off[D::ROUNDS];
#pragma unroll
  for (int r = 0; r < D::ROUNDS; ++r) {
    const int row = r * D::ROUND_ROWS + wave * 16 + (lane >> 2);
    const int c = (lane & 3) ^ code_swizzle(row);
    const bool is_a = row < T::BM;
    const int src = is_a ? min(row, rows_a - 1) : min(row - T::BM, rows_b - 1);
    c_base[r] = is_a ? qa + (size_t)m0 * kbytes : qw + (size_t)n0 * kbytes;
    c_off[r] = (uint32_t)src * kbytes + 16u * (uint32_t)c;
  }
  // scale dword of each round: LDS dword index d -> quad d / 4 (tile rows 4 quad ..), block d % 4
  const uint8_t* s_base[D::SROUNDS];
  uint32_t s_off[D::SROUNDS], s_stride[D::SROUNDS];
#pragma unroll
  for (int r = 0; r < D::SROUNDS; ++r) {
    const int d = min((r * D::WAVES + wave) * 64 + lane, D::SDW - 1);
    const int quad = d >> 2, g = d & 3;
    const bool is_a = 4 * quad < T::BM;
    const int row = is_a ? min(4 * quad, srows_a - 4) : min(4 * quad - T::BM, rows_b - 4);
    s_base[r] = is_a ? sa + m0 : sw + n0;
    s_stride[r] = is_a ? (uint32_t)ms : (uint32_t)N;
    s_off[r] = (uint32_t)g * s_stride[r] + (uint32_t)row;
  }

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // byte of the lane's row in a scale dword: result byte 0 from the block-h dword, byte 1 from
  // the block-(2 + h) dword
  const uint32_t psel = (uint32_t)(l32 & 3) | ((uint32_t)(4 + (l32 & 3)) << 8) | 0x0C0C0000u;

  // K-step kt covers 4 scale blocks: block rows 4 kt .. 4 kt + 3 of the scale tensors.
  if constexpr (PF) {
    static_assert((S - 1) * D::LOADS < 64, "vmcnt range");
    // K-steps 0 .. S - 1 fill every slot up front (the last K-step repeated where there are fewer)
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int kj = min(j, nkt - 1);
      dma_issue<D>(lds + j * D::STAGE, wave, (uint32_t)kj * (BK / 2), (size_t)kj * (BK / 32), c_base, c_off, s_base,
                   s_off, s_stride);
    }
    vm_wait_barrier<(S - 1) * D::LOADS>();  // K-step 0 has landed
    uint32_t sA0[FM][2], sB0[FN][2], sA1[FM][2], sB1[FN][2];
    i32x4_t cA0[2][FM], cB0[2][FN], cA1[2][FM], cB1[2][FN];
    mx_read_raw<T, D>(lds, wm, wn, l32, h, sA0, sB0, cA0, cB0);
    int kt = 0, sl = 0;
    for (; kt + 1 < nkt; kt += 2) {
      mx_pf_step<T, D, S>(kt, sl, nkt, lds, acc, wave, wm, wn, l32, h, psel, c_base, c_off, s_base, s_off, s_stride,
                          sA0, sB0, cA0, cB0, sA1, sB1, cA1, cB1);
      sl = sl == S - 1 ? 0 : sl + 1;
      mx_pf_step<T, D, S>(kt + 1, sl, nkt, lds, acc, wave, wm, wn, l32, h, psel, c_base, c_off, s_base, s_off,
                          s_stride, sA1, sB1, cA1, cB1, sA0, sB0, cA0, cB0);
      sl = sl == S - 1 ? 0 : sl + 1;
    }
    if (kt < nkt)
      mx_pf_step<T, D, S>(kt, sl, nkt, lds, acc, wave, wm, wn, l32, h, psel, c_base, c_off, s_base, s_off, s_stride,
                          sA0, sB0, cA0, cB0, sA1, sB1, cA1, cB1);
    vm_wait_barrier<0>();
    epilogue<T, LORA>(acc, lds, t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias, y);
    return;
  }

  // Interleaved loop: the barrier of K-step kt sits between its two halves.  Before it, the first
  // half's matrix instructions run while the second half's codes are read and K-step kt + S - 1 is
  // fetched; after it, the second half runs while the scales and first-half codes of kt + 1 are read.
  // Past the last K-step the last one is reloaded and a stale slot is read (values unused), so
  // every step issues the same loads and waits on the same vmcnt.
#pragma unroll
  for (int j = 0; j < S - 1; ++j) {
    const int kj = min(j, nkt - 1);
    dma_issue<D>(lds + j * D::STAGE, wave, (uint32_t)kj * (BK / 2), (size_t)kj * (BK / 32), c_base, c_off, s_base,
                 s_off, s_stride);
  }
  vm_wait_barrier<(S - 2) * D::LOADS>();  // K-step 0 has landed
  uint32_t qA[FM][2], qB[FN][2];
  i32x4_t c0A[FM], c0B[FN], c1A[FM], c1B[FN];
  mx_read_scales<T, D>(lds, wm, wn, l32, h, qA, qB);
  mx_read_codes<T, D>(lds, wm, wn, l32, h, 0, c0A, c0B);
  int slot = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    uint32_t sA[FM], sB[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sA[i] = __builtin_amdgcn_perm(qA[i][1], qA[i][0], psel);
#pragma unroll
    for (int j = 0; j < FN; ++j) sB[j] = __builtin_amdgcn_perm(qB[j][1], qB[j][0], psel);
    const uint8_t* cur = lds + slot * D::STAGE;
    mx_mma_half<FM, FN, 0>(acc, sA, sB, c0A, c0B);
    mx_read_codes<T, D>(cur, wm, wn, l32, h, 1, c1A, c1B);
    const int slot2 = slot == 0 ? S - 1 : slot - 1;  // read in K-step kt - 1, free since its barrier
    const int kn = min(kt + S - 1, nkt - 1);
    dma_issue<D>(lds + slot2 * D::STAGE, wave, (uint32_t)kn * (BK / 2), (size_t)kn * (BK / 32), c_base, c_off,
                 s_base, s_off, s_stride);
#pragma unroll
    for (int g = 0; g < FM * FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // direct load
    }
    __builtin_amdgcn_sched_barrier(0);
    vm_wait_barrier<(S - 2) * D::LOADS>();  // K-step kt + 1 has landed; slot kt is read
    __builtin_amdgcn_sched_barrier(0);
    slot = slot == S - 1 ? 0 : slot + 1;
    const uint8_t* nxt = lds + slot * D::STAGE;
    mx_mma_half<FM, FN, 1>(acc, sA, sB, c1A, c1B);
    mx_read_scales<T, D>(nxt, wm, wn, l32, h, qA, qB);
    mx_read_codes<T, D>(nxt, wm, wn, l32, h, 0, c0A, c0B);
#pragma unroll
    for (int g = 0; g < FM * FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
    }
  }
  vm_wait_barrier<0>();
  epilogue<T, LORA>(acc, lds, t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias, y);
}

template <int WAVES_M, int WAVES_N, int FM, int FN, int S = 3, bool PF = false>
hipError_t launch_mx_tile(int rb, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora, int parts,
                          const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                          const uint16_t* wts, const uint16_t* bias, int M, int N, int K, int R, int ms, uint16_t* y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  dim3 grid((unsigned)(((N + T::BN - 1) / T::BN) * ((M + T::BM - 1) / T::BM)));
  dim3 block(T::THREADS);
  if (rb > 0)
    gemm_mx_kernel<WAVES_M, WAVES_N, FM, FN, S, PF, true><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, ms, y);
  else
    gemm_mx_kernel<WAVES_M, WAVES_N, FM, FN, S, PF, false><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, ms, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const void* qact, const void* ascales, const float* lora, int lora_parts,
                          const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                          const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                          int64_t ms, void* y, hipStream_t stream) {
  const int rb = (int)((R + 15) / 16);
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto bs = static_cast<const uint16_t*>(bias);
  auto yp = static_cast<uint16_t*>(y);
  const int m = (int)M, n = (int)N, k = (int)K, r = (int)R, s = (int)ms;
  // batches of at most 16 rows stream the weights (W4A4_SKINNY_PATH=tiled keeps the tiles)
  const char* sp = test_hook("W4A4_SKINNY_PATH");
  if (!(sp && !strcmp(sp, "tiled")) && skinny_mx_supported(M, K, R, lora_parts))
    return launch_gemm_skinny_mx(qact, ascales, lora, lora_parts, qweight, wscales, proj_up, wcscales, wtscale, bias, M,
                                 N, K, R, ms, y, stream);
  // 16-wave 256 x 256 tiles (each wave 64 x 64: four waves per SIMD hide each other's scale
  // permutes, LDS reads and barrier waits) unless 4-wave 128 x 128 tiles need fewer rounds of
  // 256 tiles by more than the measured per-tile time ratio (2.4: 41 vs 17 us at K = 3072);
  // W4A4_GEMM_TILE=4x4x2x2, 2x4x4x2 (8 waves of 128 x 64), 2x2x4x4 (4 waves of 128 x 128 with
  // register prefetch: half the LDS reads, but measured slower) or 2x2x2x2 forces one
  const char* forced = test_hook("W4A4_GEMM_TILE");
  const int64_t rounds256 = ((M + 255) / 256 * ((N + 255) / 256) + 255) / 256;
  const int64_t rounds128 = ((M + 127) / 128 * ((N + 127) / 128) + 255) / 256;
  const bool big = forced ? !strcmp(forced, "4x4x2x2") : 2.4 * (double)rounds256 <= (double)rounds128;
  if (forced && !strcmp(forced, "2x2x4x4"))
    return launch_mx_tile<2, 2, 4, 4, 3, true>(rb, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, s,
                                               yp);
  if (forced && !strcmp(forced, "2x4x4x2"))
    return launch_mx_tile<2, 4, 4, 2>(rb, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, s, yp);
  if (big) return launch_mx_tile<4, 4, 2, 2>(rb, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, s, yp);
  return launch_mx_tile<2, 2, 2, 2>(rb, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, s, yp);
}

}  // namespace w4a4
