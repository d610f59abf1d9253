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
// the f32 accumulator.  The kernel stages the packed codes and the scales
// (converted once to f16 while staging) through LDS, decodes in registers
// with the hardware E2M1->f16 convert plus one packed f16 multiply, and issues
// v_mfma_f32_32x32x16_f16.  Only the f32 accumulation order differs from the
// exact sum.
//
// Tiling: a workgroup of WAVES_M x WAVES_N waves computes a BM x BN tile; a
// wave owns FM x FN blocks of 32 x 32.  K advances 128 columns (8 groups) per
// LDS stage, double-buffered.  Within a stage, lane half h (lane / 32) owns
// K-columns [64h, 64h + 64); MFMA sub-step kk feeds columns 64h + 8kk .. +8
// into the instruction's k-slots 8h .. 8h+8.  A and W use the same mapping,
// so the contraction covers every column exactly once.  The decode work per
// MFMA is (FM + FN) / (FM * FN) eight-element decodes, which is why the large
// tiles (4 x 4 and 4 x 3 blocks per wave) are used for the DiT shapes.
//
// Epilogue: acc *= wcscales[n] * wtscale; the rank-R correction is
// accumulated on the matrix cores (bf16 32x32x16, L split into bf16 hi + lo
// parts, proj_up exact in bf16); the tile is rounded to bf16 (nearest even),
// transposed through LDS and written with 16-byte row-contiguous stores.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int BK = 128;            // K columns per stage (8 groups of 16)
constexpr int CODE_STRIDE = 80;    // LDS bytes per code row: 64 data + 16 pad (conflict-free b128 reads)
constexpr int SCALE_STRIDE = 24;   // LDS bytes per scale row: 8 f16 + 8 pad (conflict-free b64 reads)

template <int WAVES_M, int WAVES_N, int FM, int FN>
struct Tile {
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;
  static constexpr int ROWS = BM + BN;  // A rows then B rows in LDS
  static constexpr int CHUNKS = ROWS * 4;  // 16-byte code chunks per stage
  static_assert(CHUNKS % THREADS == 0, "code chunks must split evenly over the threads");
  static constexpr int CHUNKS_PER_THREAD = CHUNKS / THREADS;
  static constexpr int SCALE_ROWS_PER_THREAD = (ROWS + THREADS - 1) / THREADS;
  static constexpr int STAGE_BYTES = ROWS * (CODE_STRIDE + SCALE_STRIDE);
  static constexpr int OUT_BYTES = BM * BN * 2;  // bf16 tile for the transposed store
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > OUT_BYTES ? 2 * STAGE_BYTES : OUT_BYTES);
};

template <class T, bool VEC16>
struct Stager {
  u32x4_t codes[T::CHUNKS_PER_THREAD];
  uint32_t sc[T::SCALE_ROWS_PER_THREAD][2];  // 8 raw e4m3 bytes per staged row

  // Branch-free: every load reads a valid address (row 0 / group 0 when out of range) and the
  // value is zeroed afterwards, so all loads issue back to back with a single wait at the use.
  __device__ __forceinline__ void load(const uint8_t* __restrict__ qa, const uint8_t* __restrict__ qw,
                                       const uint8_t* __restrict__ sa, const uint8_t* __restrict__ sw, int M, int N,
                                       int m0, int n0, int kt, int kbytes, int groups, int t) {
    const int kb0 = kt * (BK / 2);
#pragma unroll
    for (int j = 0; j < T::CHUNKS_PER_THREAD; ++j) {
      const int c = t + T::THREADS * j;
      const int row = c >> 2, piece = c & 3;
      const bool is_a = row < T::BM;
      const int gr = is_a ? m0 + row : n0 + (row - T::BM);
      const int lim = is_a ? M : N;
      const uint8_t* base = is_a ? qa : qw;
      const int off = kb0 + 16 * piece;
      if (VEC16) {
        const bool ok = gr < lim && off + 16 <= kbytes;
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + (ok ? (size_t)gr * kbytes + off : 0));
        codes[j] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const bool ok_lo = gr < lim && off + 8 <= kbytes;
        const bool ok_hi = gr < lim && off + 16 <= kbytes;
        u32x2_t lo = *reinterpret_cast<const u32x2_t*>(base + (ok_lo ? (size_t)gr * kbytes + off : 0));
        u32x2_t hi = *reinterpret_cast<const u32x2_t*>(base + (ok_hi ? (size_t)gr * kbytes + off + 8 : 0));
        codes[j] = u32x4_t{ok_lo ? lo[0] : 0u, ok_lo ? lo[1] : 0u, ok_hi ? hi[0] : 0u, ok_hi ? hi[1] : 0u};
      }
    }
    const int g0 = kt * (BK / 16);
#pragma unroll
    for (int j = 0; j < T::SCALE_ROWS_PER_THREAD; ++j) {
      const int row = t + T::THREADS * j;
      const bool is_a = row < T::BM;
      const int gr = is_a ? m0 + row : n0 + (row - T::BM);
      const int lim = is_a ? M : N;
      const uint8_t* s = is_a ? sa : sw;
      const bool row_ok = row < T::ROWS && gr < lim;
      uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const bool ok = row_ok && g0 + g < groups;
        uint32_t b = s[ok ? (size_t)(g0 + g) * lim + gr : 0];
        b = ok ? b : 0u;
        if (g < 4) w0 |= b << (8 * g); else w1 |= b << (8 * (g - 4));
      }
      sc[j][0] = w0;
      sc[j][1] = w1;
    }
  }

  __device__ __forceinline__ void store(uint8_t* __restrict__ stage, int t) const {
    uint8_t* codes_lds = stage;
    uint8_t* scale_lds = stage + T::ROWS * CODE_STRIDE;
#pragma unroll
    for (int j = 0; j < T::CHUNKS_PER_THREAD; ++j) {
      const int c = t + T::THREADS * j;
      *reinterpret_cast<u32x4_t*>(codes_lds + (c >> 2) * CODE_STRIDE + 16 * (c & 3)) = codes[j];
    }
#pragma unroll
    for (int j = 0; j < T::SCALE_ROWS_PER_THREAD; ++j) {
      const int row = t + T::THREADS * j;
      if (row < T::ROWS) {
        u32x2_t lo, hi;
        lo[0] = e4m3x2_to_h2bits(sc[j][0]);
        lo[1] = e4m3x2_to_h2bits(sc[j][0] >> 16);
        hi[0] = e4m3x2_to_h2bits(sc[j][1]);
        hi[1] = e4m3x2_to_h2bits(sc[j][1] >> 16);
        *reinterpret_cast<u32x2_t*>(scale_lds + row * SCALE_STRIDE) = lo;
        *reinterpret_cast<u32x2_t*>(scale_lds + row * SCALE_STRIDE + 8) = hi;
      }
    }
  }
};

template <int WAVES_M, int WAVES_N, int FM, int FN, bool VEC16, int RB>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::LDS_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  const int n0 = (int)(blockIdx.x % tiles_n) * T::BN;
  const int m0 = (int)(blockIdx.x / tiles_n) * T::BM;
  const int kbytes = K / 2;
  const int groups = K / 16;
  const int nkt = (K + BK - 1) / BK;

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Stager<T, VEC16> st;
  st.load(qa, qw, sa, sw, M, N, m0, n0, 0, kbytes, groups, t);
  st.store(lds, t);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) st.load(qa, qw, sa, sw, M, N, m0, n0, kt + 1, kbytes, groups, t);
    const uint8_t* cur = lds + (kt & 1) * T::STAGE_BYTES;
    const uint8_t* codes_lds = cur;
    const uint8_t* scale_lds = cur + T::ROWS * CODE_STRIDE;

    // scales for this stage: groups 4h .. 4h+3 of each fragment row, as f16
    uint32_t sA[FM][2], sB[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * FM * 32 + i * 32 + l32;
      u32x2_t v = *reinterpret_cast<const u32x2_t*>(scale_lds + row * SCALE_STRIDE + 8 * h);
      sA[i][0] = v[0]; sA[i][1] = v[1];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = T::BM + wn * FN * 32 + j * 32 + l32;
      u32x2_t v = *reinterpret_cast<const u32x2_t*>(scale_lds + row * SCALE_STRIDE + 8 * h);
      sB[j][0] = v[0]; sB[j][1] = v[1];
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4_t cA[FM], cB[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * FM * 32 + i * 32 + l32;
        cA[i] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h + 16 * half);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = T::BM + wn * FN * 32 + j * 32 + l32;
        cB[j] = *reinterpret_cast<const u32x4_t*>(codes_lds + row * CODE_STRIDE + 32 * h + 16 * half);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = 4 * half + q;  // group within the lane's half: kk / 2
        const int g = kk >> 1;
        half8_t av[FM], bv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) av[i] = decode8(cA[i][q], scale_pair(sA[i][g >> 1], g & 1));
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = decode8(cB[j][q], scale_pair(sB[j][g >> 1], g & 1));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) st.store(lds + ((kt + 1) & 1) * T::STAGE_BYTES, t);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------------------
  // All loads below read clamped, valid addresses and zero out-of-range values (branch-free).
  const float ts = bf16_bits_to_f32(wts[0]);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * FN * 32 + j * 32 + l32;
    const float c = bf16_bits_to_f32(wcs[n < N ? n : 0]) * ts;
    const float cs = n < N ? c : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= cs;
  }
  if (RB > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      bf16x8_t pv[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * FN * 32 + j * 32 + l32;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = rb * 16 + 8 * h + e;
          const bool ok = n < N && r < R;
          const uint32_t b = pu[ok ? (size_t)n * R + r : 0];
          pv[j][e] = bf16_from_bits(ok ? b : 0u);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * FM * 32 + i * 32 + l32;
        bf16x8_t lhi, llo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = rb * 16 + 8 * h + e;
          const bool ok = m < M && r < R;
          const float f0 = lora[ok ? (size_t)m * R + r : 0];
          const float f = ok ? f0 : 0.0f;
          const uint32_t hb = f32_to_bf16_bits(f);
          lhi[e] = bf16_from_bits(hb);
          llo[e] = bf16_from_bits(f32_to_bf16_bits(f - bf16_bits_to_f32(hb)));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lhi, pv[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(llo, pv[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  // bf16 tile -> LDS (row-major BM x BN), then 16-byte row-contiguous global stores.
  uint16_t* out_lds = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = wn * FN * 32 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * FM * 32 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        out_lds[row * T::BN + col] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  __syncthreads();
  constexpr int VEC_PER_ROW = T::BN / 8;  // 8 bf16 per 16-byte store
  const bool n_vec = (N % 8) == 0;
  for (int v = t; v < T::BM * VEC_PER_ROW; v += T::THREADS) {
    const int row = v / VEC_PER_ROW, cv = v % VEC_PER_ROW;
    const int m = m0 + row, n = n0 + cv * 8;
    if (m >= M || n >= N) continue;
    const u32x4_t val = *reinterpret_cast<const u32x4_t*>(out_lds + row * T::BN + cv * 8);
    uint16_t* dst = y + (size_t)m * N + n;
    if (n_vec && n + 8 <= N && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
      *reinterpret_cast<u32x4_t*>(dst) = val;
    } else {
      const uint16_t* s16 = out_lds + row * T::BN + cv * 8;
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = s16[e];
    }
  }
}

template <int WAVES_M, int WAVES_N, int FM, int FN, bool VEC16>
hipError_t launch_rb(int rb, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora,
                     const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                     const uint16_t* wts, int M, int N, int K, int R, uint16_t* y) {
  using T = Tile<WAVES_M, WAVES_N, FM, FN>;
  dim3 grid((unsigned)(((N + T::BN - 1) / T::BN) * ((M + T::BM - 1) / T::BM)));
  dim3 block(T::THREADS);
#define W4A4_GEMM_LAUNCH(RBV)                                                                      \
  gemm_kernel<WAVES_M, WAVES_N, FM, FN, VEC16, RBV><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, \
                                                                            wts, M, N, K, R, y)
  switch (rb) {
    case 0: W4A4_GEMM_LAUNCH(0); break;
    case 1: W4A4_GEMM_LAUNCH(1); break;
    case 2: W4A4_GEMM_LAUNCH(2); break;
    case 3: W4A4_GEMM_LAUNCH(3); break;
    default: W4A4_GEMM_LAUNCH(4); break;
  }
#undef W4A4_GEMM_LAUNCH
  return hipGetLastError();
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_tile(int rb, bool vec16, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora,
                       const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                       const uint16_t* wts, int M, int N, int K, int R, uint16_t* y) {
  if (vec16) return launch_rb<WAVES_M, WAVES_N, FM, FN, true>(rb, st, qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y);
  return launch_rb<WAVES_M, WAVES_N, FM, FN, false>(rb, st, qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y);
}

// Number of workgroups that fill the chip in whole waves of 256 CUs, scored so that
// larger tiles win when the fill is equal.
double tile_score(int64_t M, int64_t N, int bm, int bn) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t rounds = (tiles + 255) / 256;
  const double fill = (double)tiles / (double)(rounds * 256);
  const double useful = (double)(M * N) / (double)(((M + bm - 1) / bm) * bm * ((N + bn - 1) / bn) * bn);
  const double per_mfma_decode = (double)(bm / 64 + bn / 64) / (double)((bm / 64) * (bn / 64));  // lower is better
  return fill * useful / (1.0 + 0.5 * per_mfma_decode);
}

}  // namespace

hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, const void* qweight,
                       const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                       int64_t M, int64_t N, int64_t K, int64_t R, void* y, hipStream_t stream) {
  const int rb = (int)((R + 15) / 16);
  const bool vec16 = (K % 32) == 0;
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto yp = static_cast<uint16_t*>(y);
  const int m = (int)M, n = (int)N, k = (int)K, r = (int)R;
  // candidate tiles (BM x BN): 256x256, 256x192, 256x128, 128x128; W4A4_GEMM_TILE forces one
  double s256 = tile_score(M, N, 256, 256), s192 = tile_score(M, N, 256, 192);
  double s128 = tile_score(M, N, 256, 128), s64 = tile_score(M, N, 128, 128);
  static const char* forced = getenv("W4A4_GEMM_TILE");
  if (forced) {
    const bool a = !strcmp(forced, "256x256"), b = !strcmp(forced, "256x192"), c = !strcmp(forced, "256x128"),
               d = !strcmp(forced, "128x128");
    if (a || b || c || d) { s256 = a; s192 = b; s128 = c; s64 = d; }
  }
  const double best = fmax(fmax(s256, s192), fmax(s128, s64));
  if (best == s256) return launch_tile<2, 2, 4, 4>(rb, vec16, stream, qa, sa, lora, qw, sw, pu, wc, wt, m, n, k, r, yp);
  if (best == s192) return launch_tile<2, 2, 4, 3>(rb, vec16, stream, qa, sa, lora, qw, sw, pu, wc, wt, m, n, k, r, yp);
  if (best == s128) return launch_tile<2, 2, 4, 2>(rb, vec16, stream, qa, sa, lora, qw, sw, pu, wc, wt, m, n, k, r, yp);
  return launch_tile<2, 2, 2, 2>(rb, vec16, stream, qa, sa, lora, qw, sw, pu, wc, wt, m, n, k, r, yp);
}

}  // namespace w4a4
