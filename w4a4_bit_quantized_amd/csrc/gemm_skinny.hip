// Weight-streaming block-scaled FP4 GEMM for small batches (M <= 32), gfx950.
//
// Same result as the tiled GEMM ("SVDQuant W4A4" page, "Runtime support": NVFP4
// GEMM then the BF16 rank correction):
//   y[m,n] = bf16( sum_k A[m,k] W[n,k] * wcscales[n] * wtscale + sum_r L[m,r] proj_up[n,r] )
// With a handful of rows every weight byte is used once, so the layer is bound by
// streaming qweight/wscales from HBM.  Each workgroup owns 32 weight rows and all
// of K; its 8 waves split K into contiguous runs of 128-column steps and stream
// their weights straight into registers (two-step chunks, double-buffered, so
// several chunks of loads are in flight per wave).  No LDS staging is used for
// the weights.  Decoding is exact (E2M1 -> f16 convert, one f16 multiply by the
// e4m3 scale) and the products run on v_mfma_f32_16x16x32_f16 with the weights
// as the first operand, so a lane's accumulator holds 4 consecutive n of one m.
// The 8 per-wave partial sums are added in a fixed order through LDS; the
// epilogue applies wcscales * wtscale and adds the rank-R correction in float32
// (L from `parts` partial sums, added in order).
#include <cstdlib>

#include "device_common.h"
#include "w4a4.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int SK_WAVES = 8;
constexpr int SK_BN = 32;      // weight rows per workgroup (two 16-row MFMA blocks)
constexpr int SK_CHUNK = 2;    // K-steps per prefetch chunk

template <int MB>
struct SkinnyStep {
  u32x4_t w[2];          // weight codes, blocks 0/1: 32 consecutive k of row 16b + lane%16
  u32x4_t a[MB];         // activation codes
  uint32_t ws[2], as[MB];  // two e4m3 bytes (groups 2j, 2j+1) in bits 0..15
};

template <int MB, bool VEC16>
__device__ __forceinline__ void skinny_load(SkinnyStep<MB>& st, int step, bool active, const uint8_t* __restrict__ qa,
                                            const uint8_t* __restrict__ sa, const uint8_t* __restrict__ qw,
                                            const uint8_t* __restrict__ sw, int M, int N, int kbytes, int groups,
                                            int n0, int r16, int j) {
  const int kb = step * 64 + 16 * j;  // byte column of the lane's 32 k
  const bool tail = kb + 16 > kbytes;
  const bool ok = active && !tail;
  const int g_lo = min(step * 8 + 2 * j, groups - 1), g_hi = min(step * 8 + 2 * j + 1, groups - 1);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int n = min(n0 + 16 * b + r16, N - 1);
    const uint8_t* p = qw + (size_t)n * kbytes + (ok ? kb : 0);
    if (VEC16) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
      st.w[b] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    } else {
      const bool ok_hi = active && kb + 16 <= kbytes, ok_lo = active && kb + 8 <= kbytes;
      const uint8_t* q = qw + (size_t)n * kbytes;
      u32x2_t lo = *reinterpret_cast<const u32x2_t*>(q + (ok_lo ? kb : 0));
      u32x2_t hi = *reinterpret_cast<const u32x2_t*>(q + (ok_hi ? kb + 8 : 0));
      st.w[b] = u32x4_t{ok_lo ? lo[0] : 0u, ok_lo ? lo[1] : 0u, ok_hi ? hi[0] : 0u, ok_hi ? hi[1] : 0u};
    }
    st.ws[b] = (uint32_t)sw[(size_t)g_lo * N + n] | ((uint32_t)sw[(size_t)g_hi * N + n] << 8);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = min(16 * mb + r16, M - 1);
    const uint8_t* p = qa + (size_t)m * kbytes + (ok ? kb : 0);
    if (VEC16) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
      st.a[mb] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
    } else {
      const bool ok_hi = active && kb + 16 <= kbytes, ok_lo = active && kb + 8 <= kbytes;
      const uint8_t* q = qa + (size_t)m * kbytes;
      u32x2_t lo = *reinterpret_cast<const u32x2_t*>(q + (ok_lo ? kb : 0));
      u32x2_t hi = *reinterpret_cast<const u32x2_t*>(q + (ok_hi ? kb + 8 : 0));
      st.a[mb] = u32x4_t{ok_lo ? lo[0] : 0u, ok_lo ? lo[1] : 0u, ok_hi ? hi[0] : 0u, ok_hi ? hi[1] : 0u};
    }
    st.as[mb] = (uint32_t)sa[(size_t)g_lo * M + m] | ((uint32_t)sa[(size_t)g_hi * M + m] << 8);
  }
}

template <int MB>
__device__ __forceinline__ void skinny_compute(const SkinnyStep<MB>& st, float4_t (&acc)[MB][2]) {
  uint32_t wsh[2], ash[MB];
#pragma unroll
  for (int b = 0; b < 2; ++b) wsh[b] = e4m3x2_to_h2bits(st.ws[b]);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ash[mb] = e4m3x2_to_h2bits(st.as[mb]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // 8 consecutive k of the lane's 32; group 2j + q/2
    half8_t wv[2], av[MB];
#pragma unroll
    for (int b = 0; b < 2; ++b) wv[b] = decode8(st.w[b][q], scale_pair(wsh[b], q >> 1));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) av[mb] = decode8(st.a[mb][q], scale_pair(ash[mb], q >> 1));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[mb][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[b], av[mb], acc[mb][b], 0, 0, 0);
  }
}

template <int MB, bool VEC16, bool LORA>
__global__ __launch_bounds__(64 * SK_WAVES) void gemm_skinny_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  constexpr int MR = 16 * MB;  // padded rows
  __shared__ float red[SK_WAVES][MR][SK_BN];
  __shared__ float l_lds[LORA ? MR * W4A4_MAX_RANK : 1];
  __shared__ float p_lds[LORA ? SK_BN * (W4A4_MAX_RANK + 1) : 1];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, j = lane >> 4;
  const int n0 = blockIdx.x * SK_BN;
  const int kbytes = K / 2, groups = K / 16;
  const int nsteps = (kbytes + 63) / 64;
  const int per_wave = (nsteps + SK_WAVES - 1) / SK_WAVES;
  const int s_begin = wave * per_wave;
  const int s_end = min(s_begin + per_wave, nsteps);
  const int nchunks = (max(s_end - s_begin, 0) + SK_CHUNK - 1) / SK_CHUNK;

  float4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[mb][b] = float4_t{0.f, 0.f, 0.f, 0.f};

  SkinnyStep<MB> buf0[SK_CHUNK], buf1[SK_CHUNK];
  auto load_chunk = [&](SkinnyStep<MB>(&dst)[SK_CHUNK], int c) {
#pragma unroll
    for (int i = 0; i < SK_CHUNK; ++i) {
      const int s = s_begin + c * SK_CHUNK + i;
      skinny_load<MB, VEC16>(dst[i], s, s < s_end, qa, sa, qw, sw, M, N, kbytes, groups, n0, r16, j);
    }
  };
  auto compute_chunk = [&](const SkinnyStep<MB>(&src)[SK_CHUNK]) {
#pragma unroll
    for (int i = 0; i < SK_CHUNK; ++i) skinny_compute<MB>(src[i], acc);
  };
  if (nchunks > 0) load_chunk(buf0, 0);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) load_chunk(buf1, c + 1);
    compute_chunk(buf0);
    if (c + 1 < nchunks) {
      if (c + 2 < nchunks) load_chunk(buf0, c + 2);
      compute_chunk(buf1);
    }
  }

  // per-wave partials -> LDS: lane holds m = 16mb + lane%16, n = 16b + 4j + e
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][16 * mb + r16][16 * b + 4 * j + e] = acc[mb][b][e];
  if (LORA) {
    // L[m, r] = sum of the parts, in order; proj_up rows of this workgroup as float32
    for (int i = t; i < MR * R; i += 64 * SK_WAVES) {
      const int m = i / R, r = i % R;
      float s = 0.0f;
      if (m < M)
        for (int p = 0; p < parts; ++p) s += lora[(size_t)p * M * R + (size_t)m * R + r];
      l_lds[m * W4A4_MAX_RANK + r] = s;
    }
    for (int i = t; i < SK_BN * R; i += 64 * SK_WAVES) {
      const int n = i / R, r = i % R;
      const int nn = min(n0 + n, N - 1);
      p_lds[n * (W4A4_MAX_RANK + 1) + r] = bf16_bits_to_f32(pu[(size_t)nn * R + r]);
    }
  }
  __syncthreads();
  const float ts = bf16_bits_to_f32(wts[0]);
  for (int i = t; i < MR * SK_BN; i += 64 * SK_WAVES) {
    const int m = i / SK_BN, n = i % SK_BN;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < SK_WAVES; ++w) s += red[w][m][n];
    const int gn = n0 + n;
    if (m >= M || gn >= N) continue;
    float v = s * (bf16_bits_to_f32(wcs[gn]) * ts);
    if (LORA) {
      float l = 0.0f;
      for (int r = 0; r < R; ++r) l = __builtin_fmaf(l_lds[m * W4A4_MAX_RANK + r], p_lds[n * (W4A4_MAX_RANK + 1) + r], l);
      v += l;
    }
    y[(size_t)m * N + gn] = (uint16_t)f32_to_bf16_bits(v);
  }
}

template <int MB, bool VEC16>
hipError_t launch_mb(bool lora_on, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora, int parts,
                     const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs, const uint16_t* wts,
                     int M, int N, int K, int R, uint16_t* y) {
  dim3 grid((unsigned)((N + SK_BN - 1) / SK_BN)), block(64 * SK_WAVES);
  if (lora_on)
    gemm_skinny_kernel<MB, VEC16, true><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, M, N, K, R, y);
  else
    gemm_skinny_kernel<MB, VEC16, false><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, M, N, K, R, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const void* qact, const void* ascales, const float* lora, int lora_parts,
                              const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                              const void* wtscale, int64_t M, int64_t N, int64_t K, int64_t R, void* y,
                              hipStream_t stream) {
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto yp = static_cast<uint16_t*>(y);
  const bool vec16 = (K % 32) == 0, lo = R > 0;
  const int m = (int)M, n = (int)N, k = (int)K, r = (int)R;
  if (M <= 16) {
    if (vec16) return launch_mb<1, true>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, m, n, k, r, yp);
    return launch_mb<1, false>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, m, n, k, r, yp);
  }
  if (vec16) return launch_mb<2, true>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, m, n, k, r, yp);
  return launch_mb<2, false>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, m, n, k, r, yp);
}

}  // namespace w4a4
