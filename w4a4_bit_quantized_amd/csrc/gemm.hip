// Block-scaled FP4 GEMM with the fused low-rank epilogue (gfx950).
//
// Computes ("SVDQuant W4A4" page, "Runtime support": NVFP4 GEMM followed by
// the BF16 rank correction; "Checkpoint contract": qweight, wscales,
// proj_up, wcscales, wtscale):
//   y[m,n] = bf16( sum_k A[m,k] W[n,k] * wcscales[n] * wtscale + sum_r L[m,r] proj_up[n,r] )
//   A[m,k] = e2m1(qact[m,k]) * e4m3(ascales[k/16, m]),  W[n,k] likewise.
//
// Matrix-core route.  gfx950's scaled FP4 MFMA applies one power-of-two
// (E8M0) scale per 32 K-elements, but the contract carries one e4m3 scale
// (4 significant bits) per 16: neither the granularity nor the mantissa fits.
// Each dequantized operand e2m1 * e4m3 has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in f16, and every product is exact in
// the f32 accumulator.  The kernels stage the packed codes and the e4m3 scales
// through LDS, widen each scale pair to f16 and decode in registers with the
// hardware E2M1->f16 convert plus one packed f16 multiply, and issue
// v_mfma_f32_32x32x16_f16.  Only the f32 accumulation order differs from the
// exact sum.
//
// Tiling: a workgroup of WAVES_M x WAVES_N waves computes a BM x BN tile; a wave owns FM x FN
// blocks of 32 x 32.  K advances 128 columns (8 groups) per LDS stage.  The main kernels load
// each K-step straight into LDS (global_load_lds, three stages, K-step kt + 2 in flight while
// kt is computed); other shapes use a register-staged two-stage pipeline.  Within a stage,
// lane half h (lane / 32) owns K-columns [64h, 64h + 64); MFMA sub-step kk feeds columns
// 64h + 8kk .. +8 into the instruction's k-slots 8h .. 8h+8.  A and W use the same mapping,
// so the contraction covers every column exactly once.  The decode work per MFMA is
// (FM + FN) / (FM * FN) eight-element decodes, which is why the large tiles (4 x 2 and 2 x 3
// blocks per wave, 8 waves) are used for the DiT shapes.
//
// Epilogue: acc *= wcscales * wtscale; the rank-R correction is accumulated on the matrix
// cores (bf16 32x32x16, L split into bf16 hi + lo parts, proj_up exact in bf16); values are
// rounded to bf16 (nearest even) and, when y rows are whole 16-byte runs, pass through a
// per-wave LDS region so that each lane stores 16 contiguous bytes.  The epilogue operands of
// the tile (L summed over its partial sums, proj_up, wcscales * wtscale, bias) are first
// staged in LDS with coalesced loads.  By default the direct-load kernel is persistent: one
// workgroup per CU walks its tiles and fetches the next tile's first K-steps during the
// epilogue (gemm_dma_persist_kernel).
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace w4a4 {

// Compute units of the current device (cached per device; concurrent first calls store the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

// Global -> register -> LDS staging of one K-step.  Per-thread offsets are loop invariant;
// each K-step only moves the uniform base pointers.  Rows past M (or N) read a clamped valid
// row: they feed only output rows (columns) that are never stored.  Columns past K, which
// would mix into valid outputs, are zeroed in the one partial K-step.
template <class T, bool VEC16>
struct Stager {
  uint32_t a_off[T::A_CPT], b_off[T::B_CPT];  // row * kbytes + 16 * piece within the tile
  uint32_t s_a[T::SA_PT], s_b[T::SB_PT];      // group * rows_total + first row of the quad (clamped)
  u32x4_t a_codes[T::A_CPT], b_codes[T::B_CPT];
  uint32_t a_sc[T::SA_PT], b_sc[T::SB_PT];    // 4 raw e4m3 bytes: one group, 4 consecutive rows

  // Scale words: index i = group * (rows / 4) + quad, so consecutive threads read consecutive
  // bytes of one group row of the (K/16, rows) scale tensor.
  __device__ __forceinline__ static uint32_t scale_word_off(int i, int rows, int rows_valid, int rows_total) {
    const int quads = rows / 4;
    const int g = min(i / quads, 7);
    const int r = min(4 * (i % quads), ((rows_valid + 3) & ~3) - 4);
    return (uint32_t)(g * rows_total + r);
  }

  __device__ __forceinline__ void init(int rows_a, int rows_b, int M, int N, int kbytes, int t) {
#pragma unroll
    for (int j = 0; j < T::A_CPT; ++j) {
      const int c = t + T::THREADS * j;
      const int row = min(c >> 2, rows_a - 1);
      a_off[j] = (uint32_t)row * (uint32_t)kbytes + 16u * (uint32_t)(c & 3);
    }
#pragma unroll
    for (int j = 0; j < T::B_CPT; ++j) {
      const int c = t + T::THREADS * j;
      const int row = min(c >> 2, rows_b - 1);
      b_off[j] = (uint32_t)row * (uint32_t)kbytes + 16u * (uint32_t)(c & 3);
    }
#pragma unroll
    for (int j = 0; j < T::SA_PT; ++j) s_a[j] = scale_word_off(t + T::THREADS * j, T::BM, rows_a, M);
#pragma unroll
    for (int j = 0; j < T::SB_PT; ++j) s_b[j] = scale_word_off(t + T::THREADS * j, T::BN, rows_b, N);
  }

  template <bool TAIL>
  __device__ __forceinline__ void load_codes(const uint8_t* __restrict__ base, const uint32_t* off, u32x4_t* dst,
                                             int n, int kb0, int kbytes, int t) {
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const uint8_t* p = base + off[j];
      if (VEC16 && !TAIL) {
        dst[j] = *reinterpret_cast<const u32x4_t*>(p);
      } else {
        const int col = kb0 + 16 * ((t + T::THREADS * j) & 3);  // byte column of the chunk
        const bool ok_lo = !TAIL || col + 8 <= kbytes;
        const bool ok_hi = !TAIL || col + 16 <= kbytes;
        u32x2_t lo = *reinterpret_cast<const u32x2_t*>(ok_lo ? p : base - kb0);
        u32x2_t hi = *reinterpret_cast<const u32x2_t*>(ok_hi ? p + 8 : base - kb0);
        dst[j] = u32x4_t{ok_lo ? lo[0] : 0u, ok_lo ? lo[1] : 0u, ok_hi ? hi[0] : 0u, ok_hi ? hi[1] : 0u};
      }
    }
  }

  // SC4: every quad is 4 valid, dword-aligned rows (M and N multiples of 4); otherwise bytes.
  template <bool SC4>
  __device__ __forceinline__ static void load_scales(const uint8_t* __restrict__ base, const uint32_t* off,
                                                     uint32_t* dst, int n, int rows_valid, int rows_total,
                                                     int row0) {
#pragma unroll
    for (int j = 0; j < n; ++j) {
      if (SC4) {
        dst[j] = *reinterpret_cast<const uint32_t*>(base + off[j]);
      } else {
        const int r = (int)(off[j] % (uint32_t)rows_total);  // first row of the quad within the tile
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= (uint32_t)base[off[j] - r + min(r + e, rows_valid - 1)] << (8 * e);
        dst[j] = w;
      }
      (void)row0;
    }
  }

  template <bool TAIL, bool SC4>
  __device__ __forceinline__ void load(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ qw,
                                       const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sw, int M, int N,
                                       int m0, int n0, int rows_a, int rows_b, int kt, int kbytes, int groups,
                                       int t) {
    const int kb0 = kt * (BK / 2);
    load_codes<TAIL>(qa + (size_t)m0 * kbytes + kb0, a_off, a_codes, T::A_CPT, kb0, kbytes, t);
    load_codes<TAIL>(qw + (size_t)n0 * kbytes + kb0, b_off, b_codes, T::B_CPT, kb0, kbytes, t);
    const int g0 = kt * (BK / 16);
    if (!TAIL) {
      load_scales<SC4>(sa + (size_t)g0 * M + m0, s_a, a_sc, T::SA_PT, rows_a, M, m0);
      load_scales<SC4>(sw + (size_t)g0 * N + n0, s_b, b_sc, T::SB_PT, rows_b, N, n0);
    } else {
      // Partial K-step: groups past K read the last group (a finite scale; their codes are 0).
      tail_scales(sa, s_a, a_sc, T::SA_PT, g0, groups, rows_a, M, m0);
      tail_scales(sw, s_b, b_sc, T::SB_PT, g0, groups, rows_b, N, n0);
    }
  }

  __device__ __forceinline__ static void tail_scales(const uint8_t* __restrict__ s, const uint32_t* off, uint32_t* dst,
                                                     int n, int g0, int groups, int rows_valid, int rows_total,
                                                     int row0) {
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const int g = (int)(off[j] / (uint32_t)rows_total), r = (int)(off[j] % (uint32_t)rows_total);
      const uint8_t* b = s + (size_t)min(g0 + g, groups - 1) * rows_total + row0;
      uint32_t w = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) w |= (uint32_t)b[min(r + e, rows_valid - 1)] << (8 * e);
      dst[j] = w;
    }
  }

  __device__ __forceinline__ void store(uint8_t* __restrict__ stage, int t) const {
    uint8_t* codes_lds = stage;
    uint8_t* scale_lds = stage + T::ROWS * CODE_STRIDE;
#pragma unroll
    for (int j = 0; j < T::A_CPT; ++j) {
      const int c = t + T::THREADS * j;
      if ((T::BM * 4) % T::THREADS == 0 || c < T::BM * 4)
        *reinterpret_cast<u32x4_t*>(codes_lds + (c >> 2) * CODE_STRIDE + 16 * (c & 3)) = a_codes[j];
    }
#pragma unroll
    for (int j = 0; j < T::B_CPT; ++j) {
      const int c = t + T::THREADS * j;
      if ((T::BN * 4) % T::THREADS == 0 || c < T::BN * 4)
        *reinterpret_cast<u32x4_t*>(codes_lds + (T::BM + (c >> 2)) * CODE_STRIDE + 16 * (c & 3)) = b_codes[j];
    }
#pragma unroll
    for (int j = 0; j < T::SA_PT; ++j) {
      const int i = t + T::THREADS * j;
      if ((2 * T::BM) % T::THREADS == 0 || i < 2 * T::BM) {
        const int g = i / (T::BM / 4), r = 4 * (i % (T::BM / 4));
        *reinterpret_cast<u32x2_t*>(scale_lds + 2 * (g * T::ROWS + r)) =
            u32x2_t{e4m3x2_to_h2bits(a_sc[j]), e4m3x2_to_h2bits(a_sc[j] >> 16)};
      }
    }
#pragma unroll
    for (int j = 0; j < T::SB_PT; ++j) {
      const int i = t + T::THREADS * j;
      if ((2 * T::BN) % T::THREADS == 0 || i < 2 * T::BN) {
        const int g = i / (T::BN / 4), r = T::BM + 4 * (i % (T::BN / 4));
        *reinterpret_cast<u32x2_t*>(scale_lds + 2 * (g * T::ROWS + r)) =
            u32x2_t{e4m3x2_to_h2bits(b_sc[j]), e4m3x2_to_h2bits(b_sc[j] >> 16)};
      }
    }
  }
};

// One K-step of a wave from its operands already in registers: 8 sub-steps, each one
// v_mfma_f32_32x32x16_f16 per (i, j) fragment pair; sub-step kk + 1 is decoded while the MFMAs
// of sub-step kk run.  Sub-step kk covers K-columns 64h + 8kk .. +8 of the stage (lane half h),
// the codes of dword kk & 3 of 16-byte half kk >> 2 and the scale of group 4h + kk / 2.
template <int FM, int FN>
__device__ __forceinline__ void mma_stage(float16_t (&acc)[FM][FN], const uint32_t (&sA)[FM][2],
                                          const uint32_t (&sB)[FN][2], const u32x4_t (&cA)[2][FM],
                                          const u32x4_t (&cB)[2][FN]) {
  half8_t av[FM], bv[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) av[i] = decode8(cA[0][i][0], scale_pair(sA[i][0], 0));
#pragma unroll
  for (int j = 0; j < FN; ++j) bv[j] = decode8(cB[0][j][0], scale_pair(sB[j][0], 0));
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    half8_t an[FM], bn[FN];
    if (kk < 7) {
      const int k1 = kk + 1, hf = k1 >> 2, q = k1 & 3, g = k1 >> 1;
#pragma unroll
      for (int i = 0; i < FM; ++i) an[i] = decode8(cA[hf][i][q], scale_pair(sA[i][g >> 1], g & 1));
#pragma unroll
      for (int j = 0; j < FN; ++j) bn[j] = decode8(cB[hf][j][q], scale_pair(sB[j][g >> 1], g & 1));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[j], av[i], acc[i][j], 0, 0, 0);
    if (kk < 7) {
#pragma unroll
      for (int i = 0; i < FM; ++i) av[i] = an[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[j] = bn[j];
    }
  }
}

// The MFMA's first operand carries weight rows (output columns n) and its second operand
// activation rows (output rows m): each lane's accumulator then holds 4 consecutive n of
// one m per register quad, which is stored directly as 8 contiguous bytes of y.
template <int WAVES_M, int WAVES_N, int FM, int FN, bool VEC16, bool LORA, bool SC4>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::LDS_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  int tm, tn;
  tile_of((int)blockIdx.x, (int)gridDim.x, (M + T::BM - 1) / T::BM, tiles_n, tm, tn);
  const int n0 = tn * T::BN;
  const int m0 = tm * T::BM;
  const int kbytes = K / 2;
  const int groups = K / 16;
  const int nkt = (K + BK - 1) / BK;
  const int nfull = kbytes / (BK / 2);  // K-steps with no column past K

  Stager<T, VEC16> st;
  const int rows_a = min(T::BM, M - m0), rows_b = min(T::BN, N - n0);
  st.init(rows_a, rows_b, M, N, kbytes, t);
  if (0 < nfull) st.template load<false, SC4>(qa, qw, sa, sw, M, N, m0, n0, rows_a, rows_b, 0, kbytes, groups, t);
  else st.template load<true, SC4>(qa, qw, sa, sw, M, N, m0, n0, rows_a, rows_b, 0, kbytes, groups, t);
  st.store(lds, t);
  __syncthreads();

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      if (kt + 1 < nfull)
        st.template load<false, SC4>(qa, qw, sa, sw, M, N, m0, n0, rows_a, rows_b, kt + 1, kbytes, groups, t);
      else
        st.template load<true, SC4>(qa, qw, sa, sw, M, N, m0, n0, rows_a, rows_b, kt + 1, kbytes, groups, t);
    }
    const uint8_t* cur = lds + (kt & 1) * T::STAGE_BYTES;
    const uint8_t* codes_lds = cur;
    const uint8_t* scale_lds = cur + T::ROWS * CODE_STRIDE;

    // This stage's operands for the wave: scales of groups 4h .. 4h+3 of each fragment row
    // (f16, packed in pairs) and both halves of the packed codes.
    uint32_t sA[FM][2], sB[FN][2];
    u32x4_t cA[2][FM], cB[2][FN];
    const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(scale_lds);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * FM * 32 + i * 32 + l32;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        sA[i][p] = (uint32_t)sc16[(4 * h + 2 * p) * T::ROWS + row] | ((uint32_t)sc16[(4 * h + 2 * p + 1) * T::ROWS + row] << 16);
      cA[0][i] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h);
      cA[1][i] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h + 16);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = T::BM + wn * FN * 32 + j * 32 + l32;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        sB[j][p] = (uint32_t)sc16[(4 * h + 2 * p) * T::ROWS + row] | ((uint32_t)sc16[(4 * h + 2 * p + 1) * T::ROWS + row] << 16);
      cB[0][j] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h);
      cB[1][j] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h + 16);
    }
    mma_stage<FM, FN>(acc, sA, sB, cA, cB);
    if (more) st.store(lds + ((kt + 1) & 1) * T::STAGE_BYTES, t);
    __syncthreads();
  }

  // the K loop ended with a barrier: the stage buffers are free for the epilogue operands
  epilogue<T, LORA>(acc, lds, t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias, y);
}

// ---- three-stage variant with direct global -> LDS loads -----------------------------
// For K a multiple of 128 and M, N multiples of 4.  Everything K-step kt + 2 needs is fetched
// straight into LDS (global_load_lds: no VGPRs hold data in flight) while K-step kt is
// computed, so two K-steps of latency are covered and the only waits are the explicit ones
// ahead of each barrier.
//  * Codes: each wave instruction (dwordx4) fills 1 KB = 16 rows of 64 bytes.  Chunk c of row r
//    is placed at 16-byte position c ^ code_swizzle(r), which keeps the operand reads of 16
//    consecutive rows (one pass of a 16-byte LDS read) on distinct banks.
//  * Scales: each lane moves one dword of the (K/16, rows) scale tensor (4 consecutive rows of
//    one group); the dwords are laid out [row quad][8 groups], so a lane reads the 4 groups of
//    its half with one 16-byte read and picks its row's byte out of each dword.
// Rows past the tile's valid ones (and the padding up to whole instructions) read clamped
// valid rows and are never stored.
template <class T>
struct DmaTile {
  static constexpr int WAVES = T::WM * T::WN;
  static constexpr int ROUND_ROWS = 16 * WAVES;  // code rows one instruction per wave covers
  static constexpr int ROUNDS = (T::ROWS + ROUND_ROWS - 1) / ROUND_ROWS;
  static constexpr int SDW = 2 * T::ROWS;        // scale dwords per K-step: ROWS/4 quads x 8 groups
  static constexpr int SROUNDS = (SDW + 64 * WAVES - 1) / (64 * WAVES);
  static constexpr int SCALE_OFF = ROUNDS * ROUND_ROWS * 64;
  static constexpr int STAGE = SCALE_OFF + SROUNDS * WAVES * 256;
  static constexpr int LOADS = ROUNDS + SROUNDS;  // load instructions per wave per K-step
  static constexpr int LDS_BYTES = 3 * STAGE > T::EPI_LDS ? 3 * STAGE : T::EPI_LDS;
  static_assert(T::BM % 16 == 0 && T::ROWS % 16 == 0, "whole 16-row blocks");
};

// Per-tile addresses of a wave's direct loads: the code chunk of each round (tile row clamped to
// a valid row, swizzled 16-byte chunk) and the scale dword of each round (LDS dword index d ->
// quad d / 8 of tile rows 4 quad .., group d % 8).
template <class T>
struct DmaAddr {
  using D = DmaTile<T>;
  const uint8_t* c_base[D::ROUNDS];
  uint32_t c_off[D::ROUNDS];
  const uint8_t* s_base[D::SROUNDS];
  uint32_t s_off[D::SROUNDS], s_stride[D::SROUNDS];

  __device__ __forceinline__ void set(int wave, int lane, int m0, int n0, int M, int N, uint32_t kbytes,
                                      const uint8_t* qa, const uint8_t* sa, const uint8_t* qw, const uint8_t* sw) {
    const int rows_a = min(T::BM, M - m0), rows_b = min(T::BN, N - n0);  // multiples of 4
#pragma unroll
    for (int r = 0; r < D::ROUNDS; ++r) {
      const int row = r * D::ROUND_ROWS + wave * 16 + (lane >> 2);
      const int c = (lane & 3) ^ code_swizzle(row);
      const bool is_a = row < T::BM;
      const int src = is_a ? min(row, rows_a - 1) : min(row - T::BM, rows_b - 1);
      c_base[r] = is_a ? qa + (size_t)m0 * kbytes : qw + (size_t)n0 * kbytes;
      c_off[r] = (uint32_t)src * kbytes + 16u * (uint32_t)c;
    }
#pragma unroll
    for (int r = 0; r < D::SROUNDS; ++r) {
      const int d = min((r * D::WAVES + wave) * 64 + lane, D::SDW - 1);
      const int quad = d >> 3, g = d & 7;
      const bool is_a = 4 * quad < T::BM;
      const int row = is_a ? min(4 * quad, rows_a - 4) : min(4 * quad - T::BM, rows_b - 4);
      s_base[r] = is_a ? sa + m0 : sw + n0;
      s_stride[r] = is_a ? (uint32_t)M : (uint32_t)N;
      s_off[r] = (uint32_t)g * s_stride[r] + (uint32_t)row;
    }
  }
  // K-step kt's direct loads of this wave into the stage at `stage`
  __device__ __forceinline__ void issue(uint8_t* stage, int wave, int kt) const {
    dma_issue<D>(stage, wave, (uint32_t)kt * (BK / 2), (size_t)kt * (BK / 16), c_base, c_off, s_base, s_off, s_stride);
  }
};

// The K loop of one tile.  On entry K-steps 0 and 1 are in flight into slots 0 and 1, followed by
// S0 other vector-memory operations of this wave (stores of the previous tile, which complete
// in issue order with the loads); every wait counts what may still be in flight behind the
// K-step it needs.  Returns with every load landed and LDS free.
template <class T, int S0>
__device__ __forceinline__ void dma_k_loop(float16_t (&acc)[T::FRAG_M][T::FRAG_N], uint8_t* lds, const DmaAddr<T>& ad,
                                           int wave, int wm, int wn, int l32, int h, int nkt) {
  using D = DmaTile<T>;
  constexpr int FM = T::FRAG_M, FN = T::FRAG_N;
  static_assert(D::LOADS + S0 < 64, "vmcnt range");
  vm_wait_barrier<D::LOADS + S0>();  // K-step 0 has landed
  // byte of the lane's row within a scale dword, as a v_perm selector: result byte 0 from the
  // first dword, byte 1 from the second
  const uint32_t psel = (uint32_t)(l32 & 3) | ((uint32_t)(4 + (l32 & 3)) << 8) | 0x0C0C0000u;
  // e4m3 pair -> f16 pair in one exact convert (scale 1.0)
  auto scales_of = [&](const uint8_t* p, uint32_t (&sp)[2]) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
    sp[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(w[1], w[0], psel), 1.0f, false));
    sp[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(w[3], w[2], psel), 1.0f, false));
  };
  // Operand addresses: fragment and wave row offsets are multiples of 32, so a row's chunk
  // swizzle depends on l32 alone and every read is one of six per-lane bases (codes of chunk
  // pair half 0 / 1 and scales, for the wave's A and B rows) plus the slot and an immediate.
  const int sw4 = (l32 >> 2) & 3;
  const int ra = wm * FM * 32, rb = T::BM + wn * FN * 32;  // first A and B row of the wave
  const uint32_t lc0 = (uint32_t)(l32 * 64 + 16 * ((2 * h) ^ sw4)), lc1 = (uint32_t)(l32 * 64 + 16 * ((2 * h + 1) ^ sw4));
  const uint32_t lsc = (uint32_t)(D::SCALE_OFF + (l32 >> 2) * 32 + 16 * h);
  const uint32_t a0 = lc0 + ra * 64, a1 = lc1 + ra * 64, as = lsc + (ra >> 2) * 32;
  const uint32_t b0 = lc0 + rb * 64, b1 = lc1 + rb * 64, bs = lsc + (rb >> 2) * 32;
  // Every iteration issues the same loads (the last two reload the final K-step into a slot
  // nobody reads again), so every wave has the same count in flight at each wait.
  int slot = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    const int slot2 = slot == 0 ? 2 : slot - 1;  // (kt + 2) % 3: read in K-step kt - 1, now free
    ad.issue(lds + slot2 * D::STAGE, wave, min(kt + 2, nkt - 1));
    const uint8_t* cur = lds + slot * D::STAGE;
    uint32_t sA[FM][2], sB[FN][2];
    u32x4_t cA[2][FM], cB[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      scales_of(cur + as + i * 8 * 32, sA[i]);
      cA[0][i] = *reinterpret_cast<const u32x4_t*>(cur + a0 + i * 32 * 64);
      cA[1][i] = *reinterpret_cast<const u32x4_t*>(cur + a1 + i * 32 * 64);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      scales_of(cur + bs + j * 8 * 32, sB[j]);
      cB[0][j] = *reinterpret_cast<const u32x4_t*>(cur + b0 + j * 32 * 64);
      cB[1][j] = *reinterpret_cast<const u32x4_t*>(cur + b1 + j * 32 * 64);
    }
    mma_stage<FM, FN>(acc, sA, sB, cA, cB);
    // K-step kt + 1's loads were issued before K-step kt + 2's: at most the latter (and, after
    // K-step 0, the S0 older stores) are in flight
    if (S0 > 0 && kt == 0)
      vm_wait_barrier<D::LOADS + S0>();
    else
      vm_wait_barrier<D::LOADS>();
    slot = slot == 2 ? 0 : slot + 1;
  }
  vm_wait_barrier<0>();  // the last reloads land before LDS is reused
}

template <int WAVES_M, int WAVES_N, int FM, int FN, bool LORA>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_dma_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  using D = DmaTile<T>;
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
  const int nkt = K / BK;

  DmaAddr<T> ad;
  ad.set(wave, lane, m0, n0, M, N, (uint32_t)K / 2, qa, sa, qw, sw);
  ad.issue(lds, wave, 0);
  ad.issue(lds + D::STAGE, wave, nkt > 1 ? 1 : 0);

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  dma_k_loop<T, 0>(acc, lds, ad, wave, wm, wn, l32, h, nkt);
  epilogue<T, LORA>(acc, lds, t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias, y);
}

// ---- persistent form: the next tile's first K-steps load during the epilogue ---------------
// One workgroup per CU (or as many as fit) walks the tiles v = blockIdx.x, + gridDim.x, ... of
// the same grouped, XCD-aware order (gridDim.x a multiple of 8 keeps every tile of a workgroup
// on one XCD).  The epilogue operands live in a region E after stage slots 0 and 1, staged 32
// ranks at a time, so the next tile's K-steps 0 and 1 are fetched into those slots as soon as
// the K loop ends (before the operands are staged) and land while the epilogue computes.  y leaves through buffer
// stores: a chunk outside y gets an offset the hardware drops, so every wave issues exactly ST
// stores per tile (before the first tile, ST dropped ones), and each tile's first waits count
// them in: the stores drain while K-steps 0 and 1 run on the matrix cores.  Loads and stores
// of a wave complete in issue order on this target (the compiler's own waits assume the same).
// Needs whole 16-byte runs of y rows (N % 8 == 0, y 16-byte aligned) and |y| below 2^31 bytes.
template <int WAVES_M, int WAVES_N, int FM, int FN, bool LORA>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_dma_persist_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  using D = DmaTile<T>;
  using P = PersistTile<T, D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[P::LDS_BYTES];

  const int lane0 = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // uniform: wave-level addresses in scalar registers
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tiles_m = (M + T::BM - 1) / T::BM, tiles_n = (N + T::BN - 1) / T::BN;
  const int tiles = tiles_m * tiles_n;
  const int nkt = K / BK;
  const uint32_t kbytes = (uint32_t)K / 2;
  const uint32_t ybytes = (uint32_t)M * (uint32_t)N * 2u;
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(y, 0, (int)ybytes, 0x00020000);

  int v = (int)blockIdx.x;
  int tm, tn;
  tile_of(v, tiles, tiles_m, tiles_n, tm, tn);
  {
    DmaAddr<T> ad;
    ad.set(wave, lane0, tm * T::BM, tn * T::BN, M, N, kbytes, qa, sa, qw, sw);
    ad.issue(lds, wave, 0);
    ad.issue(lds + D::STAGE, wave, nkt > 1 ? 1 : 0);
  }
  // ST stores the hardware drops (offsets past y), so that the first tile's waits count the same
  // stores as every later tile's: one copy of the K loop.  Each has its own offset: identical
  // stores to one address would be merged into one by the compiler.
  drop_stores<P::ST>(yr);
  for (;;) {
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    // Lane-derived addresses are recomputed in each phase rather than hoisted out of the tile
    // loop, where the K loop's and the epilogue's would all stay live at once.
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int l32 = lane & 31, h = lane >> 5;
    DmaAddr<T> ad;
    ad.set(wave, lane, m0, n0, M, N, kbytes, qa, sa, qw, sw);
    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    dma_k_loop<T, P::ST>(acc, lds, ad, wave, wm, wn, l32, h, nkt);

    // epilogue; first the next tile's K-steps 0 and 1 go into slots 0 and 1
    asm volatile("" : "+v"(lane));
    const int vn = v + (int)gridDim.x;
    const bool more = vn < tiles;  // workgroup-uniform
    persist_epilogue<T, P, LORA>(acc, lds, wave, lane, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias, yr, [&] {
      if (more) {
        tile_of(vn, tiles, tiles_m, tiles_n, tm, tn);
        DmaAddr<T> nad;
        nad.set(wave, lane, tm * T::BM, tn * T::BN, M, N, kbytes, qa, sa, qw, sw);
        nad.issue(lds, wave, 0);
        nad.issue(lds + D::STAGE, wave, nkt > 1 ? 1 : 0);
      }
    });
    if (!more) break;
    v = vn;
  }
}

template <int WAVES_M, int WAVES_N, int FM, int FN, bool VEC16>
hipError_t launch_rb(int rb, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora, int parts,
                     const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                     const uint16_t* wts, const uint16_t* bias, int M, int N, int K, int R, uint16_t* y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  dim3 grid((unsigned)(((N + T::BN - 1) / T::BN) * ((M + T::BM - 1) / T::BM)));
  dim3 block(T::THREADS);
  const bool sc4 = (M % 4) == 0 && (N % 4) == 0 &&
                   ((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sw)) & 3) == 0;
#define W4A4_GEMM_GO(L, S) \
  gemm_kernel<WAVES_M, WAVES_N, FM, FN, VEC16, L, S><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y)
  if (rb > 0) {
    if (sc4) W4A4_GEMM_GO(true, true); else W4A4_GEMM_GO(true, false);
  } else {
    if (sc4) W4A4_GEMM_GO(false, true); else W4A4_GEMM_GO(false, false);
  }
#undef W4A4_GEMM_GO
  return hipGetLastError();
}

// Workgroups of the persistent kernel with this tile: as many as run at once (resident
// workgroups per CU x CUs, a multiple of 8 so that each workgroup's tiles stay on one XCD), at
// most one per tile; the W4A4_GEMM_GRID test hook caps it (several tiles per workgroup at small
// sizes).  0: not usable.  The occupancy is cached per kernel instantiation and device.
template <int WAVES_M, int WAVES_N, int FM, int FN, bool LORA>
int persist_grid(int tiles) {
  static std::atomic<int> occ[64];  // resident workgroups per CU + 1; 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int per_cu = occ[dev].load(std::memory_order_relaxed) - 1;
  if (per_cu < 0) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, gemm_dma_persist_kernel<WAVES_M, WAVES_N, FM, FN, LORA>, 64 * WAVES_M * WAVES_N, 0);
    per_cu = e == hipSuccess ? n : 0;
    occ[dev].store(per_cu + 1, std::memory_order_relaxed);
  }
  int g = per_cu * device_cus();
  if (g >= 8) g -= g % 8;
  if (const char* cap = test_hook("W4A4_GEMM_GRID")) {
    const int c = atoi(cap);
    if (c > 0 && c < g) g = c;
  }
  return g < tiles ? g : tiles;
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_dma(int rb, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora, int parts,
                      const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                      const uint16_t* wts, const uint16_t* bias, int M, int N, int K, int R, uint16_t* y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  const int tiles = ((N + T::BN - 1) / T::BN) * ((M + T::BM - 1) / T::BM);
  dim3 grid((unsigned)tiles);
  dim3 block(T::THREADS);
  if constexpr (!T::ROWWISE) {
    // persistent form: whole 16-byte runs of y rows, |y| addressable by a buffer offset;
    // the W4A4_GEMM_PERSIST=0 test hook keeps one workgroup per tile
    const char* pe = test_hook("W4A4_GEMM_PERSIST");
    const bool persist = (N % 8) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
                         (int64_t)M * N * 2 <= (int64_t)0x7FFFFFF0 && !(pe && !strcmp(pe, "0"));
    if (persist) {
      auto kern = rb > 0 ? gemm_dma_persist_kernel<WAVES_M, WAVES_N, FM, FN, true>
                         : gemm_dma_persist_kernel<WAVES_M, WAVES_N, FM, FN, false>;
      const int g = rb > 0 ? persist_grid<WAVES_M, WAVES_N, FM, FN, true>(tiles)
                           : persist_grid<WAVES_M, WAVES_N, FM, FN, false>(tiles);
      if (g > 0) {
        kern<<<dim3((unsigned)g), block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
        return hipGetLastError();
      }
    }
  }
  if (rb > 0)
    gemm_dma_kernel<WAVES_M, WAVES_N, FM, FN, true><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  else
    gemm_dma_kernel<WAVES_M, WAVES_N, FM, FN, false><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  return hipGetLastError();
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_tile(bool dma, int rb, bool vec16, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora,
                       int parts, const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                       const uint16_t* wts, const uint16_t* bias, int M, int N, int K, int R, uint16_t* y) {
  if (dma) return launch_dma<WAVES_M, WAVES_N, FM, FN>(rb, st, qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  if (vec16)
    return launch_rb<WAVES_M, WAVES_N, FM, FN, true>(rb, st, qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  return launch_rb<WAVES_M, WAVES_N, FM, FN, false>(rb, st, qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
}

// Score of a tile shape for an M x N problem: fill of whole waves of 256 CUs times the useful
// fraction of the padded tiles; larger tiles win ties (less staging per MFMA).
double tile_score(int64_t M, int64_t N, int bm, int bn) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t rounds = (tiles + 255) / 256;
  const double fill = (double)tiles / (double)(rounds * 256);
  const double useful = (double)(M * N) / (double)(((M + bm - 1) / bm) * bm * ((N + bn - 1) / bn) * bn);
  return fill * useful * (1.0 + 1e-3 * (double)(bm * bn) / 65536.0);
}

struct Variant {
  const char* name;  // waves_m x waves_n x fm x fn
  int wm, wn, fm, fn;
};
constexpr Variant kVariants[] = {
    {"2x2x4x4", 2, 2, 4, 4}, {"2x2x4x3", 2, 2, 4, 3}, {"2x2x4x2", 2, 2, 4, 2}, {"2x2x2x2", 2, 2, 2, 2},
    {"4x2x2x4", 4, 2, 2, 4}, {"2x4x4x2", 2, 4, 4, 2}, {"4x2x2x3", 4, 2, 2, 3},
};

}  // namespace

hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, int lora_parts,
                       const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                       const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                       hipStream_t stream) {
  if (M <= SKINNY_MAX_M && !test_hook("W4A4_GEMM_TILE"))
    return launch_gemm_skinny(qact, ascales, lora, lora_parts, qweight, wscales, proj_up, wcscales, wtscale, bias, M, N,
                              K, R, y, stream);
  const int rb = (int)((R + 15) / 16);
  const bool vec16 = (K % 32) == 0;
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto bs = static_cast<const uint16_t*>(bias);
  auto yp = static_cast<uint16_t*>(y);
  const int m = (int)M, n = (int)N, k = (int)K, r = (int)R;
  // The three-stage kernel with direct LDS loads needs whole 128-column K-steps and dword-aligned
  // scale quads; W4A4_GEMM_PATH=stage forces the register-staged kernel.
  const char* path = test_hook("W4A4_GEMM_PATH");
  const bool dma = (K % BK) == 0 && (M % 4) == 0 && (N % 4) == 0 &&
                   ((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sw)) & 3) == 0 &&
                   !(path && !strcmp(path, "stage"));
  // Pick the best-scoring variant; W4A4_GEMM_TILE (a variant name) forces one.
  const char* forced = test_hook("W4A4_GEMM_TILE");
  int best = -1;
  double best_score = -1.0;
  for (int i = 0; i < (int)(sizeof(kVariants) / sizeof(kVariants[0])); ++i) {
    const Variant& v = kVariants[i];
    // automatic choice: the 8-wave layouts (two waves per SIMD hide each other's LDS and
    // barrier waits) and the small 4-wave 128 x 128 tile
    if (strcmp(v.name, "2x4x4x2") && strcmp(v.name, "4x2x2x3") && strcmp(v.name, "2x2x2x2")) continue;
    const double sc = tile_score(M, N, v.wm * v.fm * 32, v.wn * v.fn * 32);
    if (sc > best_score) { best_score = sc; best = i; }
  }
  if (forced)
    for (int i = 0; i < (int)(sizeof(kVariants) / sizeof(kVariants[0])); ++i)
      if (!strcmp(forced, kVariants[i].name)) best = i;
#define W4A4_TILE_CASE(I, WM, WN, FM, FN) \
  case I: return launch_tile<WM, WN, FM, FN>(dma, rb, vec16, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
  switch (best) {
    W4A4_TILE_CASE(0, 2, 2, 4, 4)
    W4A4_TILE_CASE(1, 2, 2, 4, 3)
    W4A4_TILE_CASE(2, 2, 2, 4, 2)
    W4A4_TILE_CASE(3, 2, 2, 2, 2)
    W4A4_TILE_CASE(4, 4, 2, 2, 4)
    W4A4_TILE_CASE(5, 2, 4, 4, 2)
    default:
      return launch_tile<4, 2, 2, 3>(dma, rb, vec16, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
  }
#undef W4A4_TILE_CASE
}

}  // namespace w4a4
