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
// lies in [2^-10, 2688], so it is exact in f16; products are exact in the
// f32 accumulator.  The kernel therefore stages the packed codes and the
// scales (pre-converted to f16 pairs) through LDS, decodes in registers with
// the hardware E2M1->f16 convert plus one packed f16 multiply, and issues
// v_mfma_f32_32x32x16_f16.  Only the f32 accumulation order differs from the
// exact sum.
//
// Tiling: 128 x 128 output tile per workgroup (4 waves, 2 x 2, 64 x 64 each),
// K-step 128 (8 groups), double-buffered LDS.  Within a K-step, lane half h
// (lane / 32) owns K-columns [64h, 64h + 64); MFMA sub-step kk feeds columns
// 64h + 8kk .. +8 into the instruction's k-slots 8h .. 8h+8.  A and W use the
// same mapping, so the contraction is over every column exactly once.
//
// Epilogue: acc *= wcscales[n] * wtscale, then the rank-R correction is
// accumulated on the matrix cores (bf16 32x32x16, L split into bf16 hi + lo
// parts, proj_up bf16 exact), then rounded to bf16 (nearest even).
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int CODE_STRIDE = 80;   // bytes per tile row in LDS (64 data + 16 pad: conflict-free b128 reads)
constexpr int SCALE_STRIDE = 48;  // bytes per tile row of f16 scale pairs (32 data + 16 pad)
constexpr int TILE_CODE_BYTES = BM * CODE_STRIDE;
constexpr int TILE_SCALE_BYTES = BM * SCALE_STRIDE;
constexpr int STAGE_BYTES = 2 * TILE_CODE_BYTES + 2 * TILE_SCALE_BYTES;

struct Staged {
  u32x4_t a_codes[2], b_codes[2];
  uint32_t a_sc, b_sc;  // 4 scale bytes each (one group, 4 consecutive rows)
};

// Global -> registers for one K-step.  Thread t: tile row t/2, 32-byte half t%2
// of the 64-byte code row; scales: group t/32, rows 4*(t%32) .. +4.
template <bool VEC16>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ base, int rows_total, int row0, int kbyte0,
                                           int kbytes, int t, u32x4_t (&out)[2]) {
  const int r = row0 + (t >> 1);
  const int cb = kbyte0 + (t & 1) * 32;
  const uint8_t* p = base + (size_t)(r < rows_total ? r : 0) * kbytes;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int off = cb + 16 * j;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < rows_total) {
      if (VEC16) {
        if (off + 16 <= kbytes) v = *reinterpret_cast<const u32x4_t*>(p + off);
      } else {
        if (off + 8 <= kbytes) {
          u32x2_t lo = *reinterpret_cast<const u32x2_t*>(p + off);
          v[0] = lo[0]; v[1] = lo[1];
        }
        if (off + 16 <= kbytes) {
          u32x2_t hi = *reinterpret_cast<const u32x2_t*>(p + off + 8);
          v[2] = hi[0]; v[3] = hi[1];
        }
      }
    }
    out[j] = v;
  }
}

__device__ __forceinline__ uint32_t load_scales(const uint8_t* __restrict__ sc, int rows_total, int row0, int g0,
                                                int groups, int t) {
  const int g = g0 + (t >> 5);
  const int r = row0 + 4 * (t & 31);
  uint32_t w = 0u;
  if (g < groups) {
    const uint8_t* p = sc + (size_t)g * rows_total;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (r + i < rows_total) w |= (uint32_t)p[r + i] << (8 * i);
  }
  return w;
}

__device__ __forceinline__ void store_stage(uint8_t* __restrict__ lds, const Staged& s, int t) {
  uint8_t* a_codes = lds;
  uint8_t* b_codes = lds + TILE_CODE_BYTES;
  uint8_t* a_sc = lds + 2 * TILE_CODE_BYTES;
  uint8_t* b_sc = a_sc + TILE_SCALE_BYTES;
  const int r = t >> 1, half = t & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    *reinterpret_cast<u32x4_t*>(a_codes + r * CODE_STRIDE + half * 32 + 16 * j) = s.a_codes[j];
    *reinterpret_cast<u32x4_t*>(b_codes + r * CODE_STRIDE + half * 32 + 16 * j) = s.b_codes[j];
  }
  const int g = t >> 5, r0 = 4 * (t & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint32_t*>(a_sc + (r0 + i) * SCALE_STRIDE + 4 * g) = e4m3_to_h2bits((s.a_sc >> (8 * i)) & 0xFFu);
    *reinterpret_cast<uint32_t*>(b_sc + (r0 + i) * SCALE_STRIDE + 4 * g) = e4m3_to_h2bits((s.b_sc >> (8 * i)) & 0xFFu);
  }
}

template <bool VEC16, int RB>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_BYTES];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int tiles_n = (N + BN - 1) / BN;
  const int n0 = (int)(blockIdx.x % tiles_n) * BN;
  const int m0 = (int)(blockIdx.x / tiles_n) * BM;
  const int kbytes = K / 2;
  const int groups = K / 16;
  const int nkt = (K + BK - 1) / BK;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Staged st;
  load_codes<VEC16>(qa, M, m0, 0, kbytes, t, st.a_codes);
  load_codes<VEC16>(qw, N, n0, 0, kbytes, t, st.b_codes);
  st.a_sc = load_scales(sa, M, m0, 0, groups, t);
  st.b_sc = load_scales(sw, N, n0, 0, groups, t);
  store_stage(lds, st, t);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      const int kb = (kt + 1) * (BK / 2);
      load_codes<VEC16>(qa, M, m0, kb, kbytes, t, st.a_codes);
      load_codes<VEC16>(qw, N, n0, kb, kbytes, t, st.b_codes);
      st.a_sc = load_scales(sa, M, m0, (kt + 1) * (BK / 16), groups, t);
      st.b_sc = load_scales(sw, N, n0, (kt + 1) * (BK / 16), groups, t);
    }
    const uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    const uint8_t* a_codes = cur;
    const uint8_t* b_codes = cur + TILE_CODE_BYTES;
    const uint8_t* a_sc = cur + 2 * TILE_CODE_BYTES;
    const uint8_t* b_sc = a_sc + TILE_SCALE_BYTES;

    uint32_t ac[2][8], bc[2][8];
    uint32_t as_[2][4], bs_[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int ra = wm * 64 + f * 32 + l32;
      const int rb_ = wn * 64 + f * 32 + l32;
      u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(a_codes + ra * CODE_STRIDE + h * 32);
      u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(a_codes + ra * CODE_STRIDE + h * 32 + 16);
      u32x4_t b0 = *reinterpret_cast<const u32x4_t*>(b_codes + rb_ * CODE_STRIDE + h * 32);
      u32x4_t b1 = *reinterpret_cast<const u32x4_t*>(b_codes + rb_ * CODE_STRIDE + h * 32 + 16);
      u32x4_t sa4 = *reinterpret_cast<const u32x4_t*>(a_sc + ra * SCALE_STRIDE + h * 16);
      u32x4_t sb4 = *reinterpret_cast<const u32x4_t*>(b_sc + rb_ * SCALE_STRIDE + h * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ac[f][i] = a0[i]; ac[f][4 + i] = a1[i];
        bc[f][i] = b0[i]; bc[f][4 + i] = b1[i];
        as_[f][i] = sa4[i]; bs_[f][i] = sb4[i];
      }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      half8_t av[2], bv[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        av[f] = decode8(ac[f][kk], __builtin_bit_cast(half2_t, as_[f][kk >> 1]));
        bv[f] = decode8(bc[f][kk], __builtin_bit_cast(half2_t, bs_[f][kk >> 1]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_stage(lds + ((kt + 1) & 1) * STAGE_BYTES, st, t);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------------------
  const float ts = bf16_bits_to_f32(wts[0]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    const float c = n < N ? bf16_bits_to_f32(wcs[n]) * ts : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= c;
  }
  if (RB > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      bf16x8_t lhi[2], llo[2], pv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + wm * 64 + i * 32 + l32;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = rb * 16 + 8 * h + e;
          const float f = (m < M && r < R) ? lora[(size_t)m * R + r] : 0.0f;
          const uint32_t hb = f32_to_bf16_bits(f);
          lhi[i][e] = bf16_from_bits(hb);
          llo[i][e] = bf16_from_bits(f32_to_bf16_bits(f - bf16_bits_to_f32(hb)));
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = rb * 16 + 8 * h + e;
          pv[j][e] = bf16_from_bits((n < N && r < R) ? pu[(size_t)n * R + r] : 0u);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lhi[i], pv[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(llo[i], pv[j], acc[i][j], 0, 0, 0);
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (m < M && n < N) y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
    }
}

template <bool VEC16>
hipError_t launch_rb(int rb, dim3 grid, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora,
                     const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs,
                     const uint16_t* wts, int M, int N, int K, int R, uint16_t* y) {
  dim3 block(256);
  switch (rb) {
    case 0: gemm_kernel<VEC16, 0><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y); break;
    case 1: gemm_kernel<VEC16, 1><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y); break;
    case 2: gemm_kernel<VEC16, 2><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y); break;
    case 3: gemm_kernel<VEC16, 3><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y); break;
    default: gemm_kernel<VEC16, 4><<<grid, block, 0, st>>>(qa, sa, lora, qw, sw, pu, wcs, wts, M, N, K, R, y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* qact, const void* ascales, const float* lora, const void* qweight,
                       const void* wscales, const void* proj_up, const void* wcscales, const void* wtscale,
                       int64_t M, int64_t N, int64_t K, int64_t R, void* y, hipStream_t stream) {
  const int rb = (int)((R + 15) / 16);
  dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + BM - 1) / BM)));
  const bool vec16 = (K % 32) == 0;
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto yp = static_cast<uint16_t*>(y);
  if (vec16) return launch_rb<true>(rb, grid, stream, qa, sa, lora, qw, sw, pu, wc, wt, (int)M, (int)N, (int)K, (int)R, yp);
  return launch_rb<false>(rb, grid, stream, qa, sa, lora, qw, sw, pu, wc, wt, (int)M, (int)N, (int)K, (int)R, yp);
}

}  // namespace w4a4
