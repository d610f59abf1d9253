// Weight-streaming block-scaled FP4 GEMM for small batches (M <= 32), gfx950.
//
// Same result as the tiled GEMM ("SVDQuant W4A4" page, "Runtime support": NVFP4
// GEMM then the BF16 rank correction):
//   y[m,n] = bf16( sum_k A[m,k] W[n,k] * wcscales[n] * wtscale + sum_r L[m,r] proj_up[n,r] )
// With a handful of rows every weight byte is used once, so the layer is bound by
// streaming qweight/wscales from HBM.  Decoding is exact (E2M1 -> f16 convert, one f16
// multiply by the e4m3 scale) and the products run on v_mfma_f32_16x16x32_f16 with the
// weights as the first operand, so a lane's accumulator holds 4 consecutive n of one m.
// Three variants:
//   * wide (M <= 16, K <= 5120, more than 8192 columns): 64 weight rows per 1024-thread
//     workgroup, chunks of 512 K-columns staged through LDS two chunks ahead of the compute,
//     each code decoded once per workgroup;
//   * stream (M <= 16, K <= 5120, fewer columns): 32 rows per 512-thread workgroup, every
//     load of the workgroup's share issued up front, staged through LDS in two phases;
//   * registers (any K, M <= 32): 32 rows per workgroup, 8 waves split K into contiguous
//     runs of 128-column steps loaded straight into registers in the MFMA layout.
// The per-wave partial sums are added in a fixed order through LDS; the epilogue applies
// wcscales * wtscale and adds the rank-R correction in float32 (L from `parts` partial sums,
// added in order).
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "w4a4.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int SK_WAVES = 8;
constexpr int SK_BN = 32;      // weight rows per workgroup (two 16-row MFMA blocks)
constexpr int SK_MAXPARTS = 8;  // low-rank partial sums whose loads are issued together
constexpr int SK_BATCH = 5;    // K-steps whose loads are issued together

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
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
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

  // ---- epilogue operands first: their loads overlap the weight stream -------------------
  constexpr int LPT = (MR * W4A4_MAX_RANK + 64 * SK_WAVES - 1) / (64 * SK_WAVES);
  constexpr int PPT = (SK_BN * W4A4_MAX_RANK + 64 * SK_WAVES - 1) / (64 * SK_WAVES);
  float lsum[LORA ? LPT : 1];
  uint32_t pval[LORA ? PPT : 1];
  uint32_t cval = 0u;
  if (t < SK_BN) cval = wcs[min(n0 + t, N - 1)];
  if (LORA) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;  // (m, r) = (i / R, i % R)
      const int m = min(i / max(R, 1), M - 1), r = i % max(R, 1);
      const size_t at = (size_t)m * R + r;
      float v[SK_MAXPARTS];
#pragma unroll
      for (int p = 0; p < SK_MAXPARTS; ++p) v[p] = lora[(size_t)min(p, parts - 1) * M * R + at];
      float sum = 0.0f;  // the parts in order; the spare terms add +0 and change nothing
#pragma unroll
      for (int p = 0; p < SK_MAXPARTS; ++p) sum += p < parts ? v[p] : 0.0f;
      for (int p = SK_MAXPARTS; p < parts; ++p) sum += lora[(size_t)p * M * R + at];
      lsum[u] = sum;
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      const int n = min(n0 + i / max(R, 1), N - 1), r = i % max(R, 1);
      pval[u] = pu[(size_t)n * R + r];
    }
  }

  float4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[mb][b] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int s0 = s_begin; s0 < s_end; s0 += SK_BATCH) {
    SkinnyStep<MB> st[SK_BATCH];
#pragma unroll
    for (int i = 0; i < SK_BATCH; ++i)
      skinny_load<MB, VEC16>(st[i], s0 + i, s0 + i < s_end, qa, sa, qw, sw, M, N, kbytes, groups, n0, r16, j);
#pragma unroll
    for (int i = 0; i < SK_BATCH; ++i)
      if (s0 + i < s_end) skinny_compute<MB>(st[i], acc);  // wave-uniform
  }

  // per-wave partials -> LDS: lane holds m = 16mb + lane%16, n = 16b + 4j + e
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][16 * mb + r16][16 * b + 4 * j + e] = acc[mb][b][e];
  __shared__ float c_lds[SK_BN];
  if (t < SK_BN) c_lds[t] = bf16_bits_to_f32(cval) * bf16_bits_to_f32(wts[0]);
  if (LORA) {
    // L[m, r] = sum of the parts, in order; proj_up rows of this workgroup as float32
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      if (i < MR * R) l_lds[(i / R) * W4A4_MAX_RANK + i % R] = lsum[u];
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      if (i < SK_BN * R) p_lds[(i / R) * (W4A4_MAX_RANK + 1) + i % R] = bf16_bits_to_f32(pval[u]);
    }
  }
  __syncthreads();
  for (int i = t; i < MR * SK_BN; i += 64 * SK_WAVES) {
    const int m = i / SK_BN, n = i % SK_BN;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < SK_WAVES; ++w) s += red[w][m][n];
    const int gn = n0 + n;
    if (m >= M || gn >= N) continue;
    float v = s * c_lds[n];
    if (LORA) {
      float l = 0.0f;
      for (int r = 0; r < R; ++r) l = __builtin_fmaf(l_lds[m * W4A4_MAX_RANK + r], p_lds[n * (W4A4_MAX_RANK + 1) + r], l);
      v += l;
    }
    if (bias != nullptr) v += bf16_bits_to_f32(bias[gn]);
    y[(size_t)m * N + gn] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ---- streaming variant for M <= 16 (a multiple of 4), K <= 5120 (a multiple of 512) -----
// The loads follow the layout of memory: for each 256-byte chunk of a row (512 K-columns),
// thread t reads 16 bytes of weight row t / 16 at byte 16 (t % 16) (32 runs of 256 contiguous
// bytes per instruction) and 8 bytes of activation row t / 32 at byte 8 (t % 32); the first
// threads also read the chunk's wscales and ascales as dwords (4 rows of one group).  A
// workgroup issues the loads of all its chunks (its whole share of K) before any compute.  The
// chunks then pass through LDS, five at a time, to reach the MFMA layout: wave w computes a
// chunk's K-columns 64w .. 64w + 63; lane (row i = lane % 16, kg = lane / 16) takes the 8
// bytes at 32w + 8kg (16 codes, two MFMA sub-steps, one 16-group 4w + kg) of its row, for the
// activations and for both 16-row weight blocks.
constexpr int SS_CH = 256;                // bytes of a row per chunk (512 K-columns)
constexpr int SS_ROW = SS_CH + 16;        // LDS bytes per row of a chunk (16 bytes of padding)
constexpr int SS_MAXC = 10;               // chunks of K (K <= 5120), loads all issued up front
constexpr int SS_PHASE = 5;               // chunks staged in LDS per barrier
constexpr int SS_MAXPARTS = 8;            // low-rank partial sums the epilogue adds
constexpr int SS_W = 0;                               // slot layout: weight rows
constexpr int SS_S = SS_W + SK_BN * SS_ROW;           // wscales [group][32 rows]
constexpr int SS_A = SS_S + 32 * SK_BN;               // activation rows
constexpr int SS_AS = SS_A + 16 * SS_ROW;             // ascales [group][16 rows]
constexpr int SS_SLOT = SS_AS + 32 * 16;
constexpr int SS_LDS = SS_PHASE * SS_SLOT;

template <bool LORA>
__global__ __launch_bounds__(64 * SK_WAVES) void gemm_skinny_stream_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  constexpr int MR = 16;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SS_LDS];
  // after the chunk loop the same bytes hold the reduction and the epilogue operands
  float (*red)[MR][SK_BN] = reinterpret_cast<float (*)[MR][SK_BN]>(smem);
  float* l_lds = reinterpret_cast<float*>(smem + SK_WAVES * MR * SK_BN * 4);
  float* p_lds = l_lds + MR * W4A4_MAX_RANK;
  float* c_lds = p_lds + SK_BN * (W4A4_MAX_RANK + 1);
  static_assert(SK_WAVES * MR * SK_BN * 4 + (MR * W4A4_MAX_RANK + SK_BN * (W4A4_MAX_RANK + 1) + SK_BN) * 4 <= SS_LDS,
                "epilogue fits the staging area");

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int n0 = blockIdx.x * SK_BN;
  const int kbytes = K / 2;
  const int nc = kbytes / SS_CH;  // 1 .. SS_MAXC

  // ---- every load of the workgroup's share, up front (clamped past the last chunk) ------
  const uint8_t* wsrc = qw + (size_t)min(n0 + (t >> 4), N - 1) * kbytes + 16 * (t & 15);
  const uint8_t* asrc = qa + (size_t)min(t >> 5, M - 1) * kbytes + 8 * (t & 31);
  const int sg = (t >> 3) & 31, sq = t & 7;  // wscales dword of threads < 256
  const uint8_t* ssrc = sw + (size_t)sg * N + min(n0 + 4 * sq, N - 4);
  const int ag = (t >> 2) & 31, aq = t & 3;  // ascales dword of threads < 128
  const uint8_t* assrc = sa + (size_t)ag * M + min(4 * aq, M - 4);
  u32x4_t wr[SS_MAXC];
  u32x2_t ar[SS_MAXC];
  uint32_t sr[SS_MAXC], asr[SS_MAXC];
#pragma unroll
  for (int i = 0; i < SS_MAXC; ++i) {
    const int c = min(i, nc - 1);
    wr[i] = *reinterpret_cast<const u32x4_t*>(wsrc + (size_t)c * SS_CH);
    ar[i] = *reinterpret_cast<const u32x2_t*>(asrc + (size_t)c * SS_CH);
  }
  if (t < 256) {
#pragma unroll
    for (int i = 0; i < SS_MAXC; ++i) sr[i] = *reinterpret_cast<const uint32_t*>(ssrc + (size_t)min(i, nc - 1) * 32 * N);
  }
  if (t < 128) {
#pragma unroll
    for (int i = 0; i < SS_MAXC; ++i) asr[i] = *reinterpret_cast<const uint32_t*>(assrc + (size_t)min(i, nc - 1) * 32 * M);
  }

  float4_t acc[2];
  acc[0] = float4_t{0.f, 0.f, 0.f, 0.f};
  acc[1] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int a_group = 4 * wave + kg;  // 16-group of the lane within a chunk
#pragma unroll
  for (int ph = 0; ph < SS_MAXC; ph += SS_PHASE) {
    if (ph >= nc) continue;  // workgroup-uniform
    if (ph > 0) __syncthreads();  // every wave is done with the previous phase's slots
#pragma unroll
    for (int i = ph; i < ph + SS_PHASE; ++i) {
      uint8_t* slot = smem + (i - ph) * SS_SLOT;
      *reinterpret_cast<u32x4_t*>(slot + SS_W + (t >> 4) * SS_ROW + 16 * (t & 15)) = wr[i];
      *reinterpret_cast<u32x2_t*>(slot + SS_A + (t >> 5) * SS_ROW + 8 * (t & 31)) = ar[i];
      if (t < 256) *reinterpret_cast<uint32_t*>(slot + SS_S + sg * SK_BN + 4 * sq) = sr[i];
      if (t < 128) *reinterpret_cast<uint32_t*>(slot + SS_AS + ag * 16 + 4 * aq) = asr[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = ph; i < ph + SS_PHASE; ++i) {
      if (i >= nc) continue;  // workgroup-uniform
      const uint8_t* slot = smem + (i - ph) * SS_SLOT;
      const u32x2_t ac = *reinterpret_cast<const u32x2_t*>(slot + SS_A + r16 * SS_ROW + 32 * wave + 8 * kg);
      const uint32_t asb = slot[SS_AS + a_group * 16 + r16];
      const uint32_t ash = e4m3x2_to_h2bits(asb | (asb << 8));
      const half8_t a0 = decode8(ac[0], scale_pair(ash, 0));
      const half8_t a1 = decode8(ac[1], scale_pair(ash, 0));
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = 16 * b + r16;
        const u32x2_t wc = *reinterpret_cast<const u32x2_t*>(slot + SS_W + row * SS_ROW + 32 * wave + 8 * kg);
        const uint32_t wsb = slot[SS_S + a_group * SK_BN + row];
        const uint32_t wsh = e4m3x2_to_h2bits(wsb | (wsb << 8));
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(wc[0], scale_pair(wsh, 0)), a0, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(wc[1], scale_pair(wsh, 0)), a1, acc[b], 0, 0, 0);
      }
    }
  }

  // ---- epilogue operands (fetched after the stream: holding them during it would spill) ----
  constexpr int LPT = (MR * W4A4_MAX_RANK + 64 * SK_WAVES - 1) / (64 * SK_WAVES);
  constexpr int PPT = (SK_BN * W4A4_MAX_RANK + 64 * SK_WAVES - 1) / (64 * SK_WAVES);
  float lsum[LORA ? LPT : 1];
  uint32_t pval[LORA ? PPT : 1];
  const uint32_t cval = wcs[min(n0 + (t % SK_BN), N - 1)];
  if (LORA) {
    lsum[LPT - 1] = 0.0f;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      if (u > 0 && MR * R <= u * 64 * SK_WAVES) continue;  // uniform: no rows of R ranks left
      const int i = t + u * 64 * SK_WAVES;
      const size_t at = (size_t)min(i / R, M - 1) * R + i % R;
      float v[SS_MAXPARTS];
#pragma unroll
      for (int p = 0; p < SS_MAXPARTS; ++p) v[p] = lora[(size_t)min(p, parts - 1) * M * R + at];
      float sum = 0.0f;  // the parts in order; the spare terms add +0 and change nothing
#pragma unroll
      for (int p = 0; p < SS_MAXPARTS; ++p) sum += p < parts ? v[p] : 0.0f;
      lsum[u] = sum;
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      pval[u] = pu[(size_t)min(n0 + i / R, N - 1) * R + i % R];
    }
  }
  __syncthreads();  // the staging area is reused below

  // per-wave partials -> LDS: lane holds m = lane%16, n = 16b + 4 kg + e
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][r16][16 * b + 4 * kg + e] = acc[b][e];
  if (t < SK_BN) c_lds[t] = bf16_bits_to_f32(cval) * bf16_bits_to_f32(wts[0]);
  if (LORA) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      if (i < MR * R) l_lds[(i / R) * W4A4_MAX_RANK + i % R] = lsum[u];
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SK_WAVES;
      if (i < SK_BN * R) p_lds[(i / R) * (W4A4_MAX_RANK + 1) + i % R] = bf16_bits_to_f32(pval[u]);
    }
  }
  __syncthreads();
  for (int i = t; i < MR * SK_BN; i += 64 * SK_WAVES) {
    const int mm = i / SK_BN, n = i % SK_BN;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < SK_WAVES; ++w) s += red[w][mm][n];
    const int gn = n0 + n;
    if (mm >= M || gn >= N) continue;
    float v = s * c_lds[n];
    if (LORA) {
      float l = 0.0f;
      for (int r = 0; r < R; ++r) l = __builtin_fmaf(l_lds[mm * W4A4_MAX_RANK + r], p_lds[n * (W4A4_MAX_RANK + 1) + r], l);
      v += l;
    }
    if (bias != nullptr) v += bf16_bits_to_f32(bias[gn]);
    y[(size_t)mm * N + gn] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ---- wide variant for M <= 16, K <= 5120 (a multiple of 512) and many columns --------------
// One 1024-thread workgroup per 64 weight rows (four 16-row MFMA blocks) and all of K.  Chunks
// of 512 K-columns pass through LDS: per chunk, thread t loads 16 bytes of weight row t / 16,
// 4 bytes of activation row t / 64, two wscales bytes (group t / 32) and one ascales byte; the
// scales are widened to f16 pairs as they are stored.  Wave w owns the chunk's K-columns
// 32w .. 32w + 31 for all four blocks, so each activation code and each weight code of the
// tile is decoded once; lane (i = lane % 16, kg = lane / 16) takes the 8 codes at byte
// 16w + 4kg of its rows.  Loads run SW_AHEAD chunks ahead of the compute: a deeper prefetch,
// or issuing every chunk up front, delays the first chunk (the memory system serves a
// workgroup's outstanding requests together) and measured slower.  Tiles are numbered so
// that consecutive tiles run on one XCD (workgroups go to the 8 XCDs in turn) and share the
// L2 lines of wscales.  The 16 per-wave partial sums meet in LDS in a fixed order; the rank-R
// term runs on the matrix cores (L split into bf16 hi + lo parts) and is added before the
// single rounding to bf16.
constexpr int SW_WAVES = 16;
constexpr int SW_BN = 64;                            // weight rows per workgroup
constexpr int SW_AHEAD = 2;                          // chunks in flight ahead of the compute
constexpr int SW_SSTR = 80;                          // dwords per group row of staged wscales
constexpr int SW_W = 0;                              // slot: weight rows (SS_ROW bytes each)
constexpr int SW_A = SW_W + SW_BN * SS_ROW;          //       activation rows
constexpr int SW_S = SW_A + 16 * SS_ROW;             //       wscales as f16 pairs [32 groups][SW_SSTR]
constexpr int SW_AS = SW_S + 32 * SW_SSTR * 4;       //       ascales as f16 pairs [32 groups][16 rows]
constexpr int SW_SLOT = SW_AS + 32 * 16 * 4;
constexpr int SW_RED = 68;                           // floats per row of the reduction area
constexpr int SW_REDB = (SW_WAVES + 1) * 16 * SW_RED * 4;
constexpr int SW_EPI = 2 * SW_SLOT > SW_REDB ? 2 * SW_SLOT : SW_REDB;
constexpr int SW_RS = W4A4_MAX_RANK + 8;             // bf16 per staged rank row (144-byte rows)
constexpr int SW_LHI = SW_EPI;
constexpr int SW_LLO = SW_LHI + 16 * SW_RS * 2;
constexpr int SW_P = SW_LLO + 16 * SW_RS * 2;
constexpr int SW_C = SW_P + SW_BN * SW_RS * 2;
constexpr int SW_TRASH = SW_C + SW_BN * 4;           // target of lanes with nothing to store
constexpr int SW_LDS = SW_TRASH + 16;
static_assert(SW_LDS <= 160 * 1024, "LDS of one CU");

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Tile of workgroup b when workgroups are dispatched to the 8 XCDs in turn: XCD x runs a
// contiguous range of tiles.
__device__ __forceinline__ int xcd_tile(int b, int G) {
  const int q = G / 8, r = G % 8, x = b % 8, l = b / 8;
  return x < r ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

// f16 pair {s, s} of the e4m3 byte in bits 0..7 of b (exact)
__device__ __forceinline__ uint32_t e4m3_dup_h2bits(uint32_t b) {
  const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(b, false);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[0]));
}

// FULL: K == 512 * SS_MAXC, so no chunk index is clamped and chunk offsets are immediates
template <bool LORA, int RP, bool FULL>
__global__ __launch_bounds__(64 * SW_WAVES) void gemm_skinny_wide_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M, int N, int K, int R,
    uint16_t* __restrict__ y) {
  static_assert(!LORA || RP == 32 || RP == 64, "rank padded to one or two MFMA steps");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SW_LDS];
  uint16_t* l_hi = reinterpret_cast<uint16_t*>(smem + SW_LHI);
  uint16_t* l_lo = reinterpret_cast<uint16_t*>(smem + SW_LLO);
  uint16_t* p_lds = reinterpret_cast<uint16_t*>(smem + SW_P);
  float* c_lds = reinterpret_cast<float*>(smem + SW_C);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int n0 = xcd_tile(blockIdx.x, gridDim.x) * SW_BN;
  const int kbytes = K / 2;
  const int nc = FULL ? SS_MAXC : kbytes / SS_CH;  // 1 .. SS_MAXC

  // ---- epilogue operands first: the oldest loads, complete before the first chunk is used ----
  // Every load here and below is unconditional (indices clamped), so none is moved past its use.
  constexpr int RPP = RP > 0 ? RP : 1;
  constexpr int PPT = LORA ? SW_BN * RP / (64 * SW_WAVES) : 1;
  const uint32_t cval = wcs[min(n0 + (t & 63), N - 1)];
  const uint32_t tsv = wts[0];
  const int lm = t / RPP, lr = t % RPP;  // the (m, r) element of L this thread stages
  float lv[SS_MAXPARTS];
  uint32_t pval[PPT];
  if (LORA) {
    const int at = min(min(lm, M - 1) * R + min(lr, R - 1), M * R - 1);
#pragma unroll
    for (int p = 0; p < SS_MAXPARTS; ++p) lv[p] = lora[(size_t)min(p, parts - 1) * M * R + at];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SW_WAVES;
      pval[u] = pu[(size_t)min(n0 + i / RPP, N - 1) * R + min(i % RPP, R - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const uint8_t* wsrc = qw + (size_t)min(n0 + (t >> 4), N - 1) * kbytes + 16 * (t & 15);
  const uint8_t* asrc = qa + (size_t)min(t >> 6, M - 1) * kbytes + 4 * (t & 63);
  const uint32_t soff = (uint32_t)((t >> 5) * N + min(n0 + 2 * (t & 31), N - 2));  // within a chunk's groups
  const uint32_t asoff = (uint32_t)(((t & 511) >> 4) * M + min(t & 15, M - 1));
  u32x4_t wr[SS_MAXC];
  uint32_t ar[SS_MAXC], sr[SS_MAXC], asr[SS_MAXC];
// chunk j's loads (chunks past the last reload it); the scheduling barrier keeps chunks in order
#define W4A4_SW_ISSUE(j)                                                              \
  do {                                                                                \
    const int c_ = FULL ? (j) : min((j), nc - 1);                                     \
    wr[(j)] = *reinterpret_cast<const u32x4_t*>(wsrc + c_ * SS_CH);                   \
    ar[(j)] = *reinterpret_cast<const uint32_t*>(asrc + c_ * SS_CH);                  \
    sr[(j)] = *reinterpret_cast<const uint16_t*>(sw + (size_t)c_ * 32 * N + soff);    \
    asr[(j)] = (sa + (size_t)c_ * 32 * M)[asoff];                                     \
    __builtin_amdgcn_sched_barrier(0);                                                \
  } while (0)
#pragma unroll
  for (int j = 0; j < SW_AHEAD; ++j) W4A4_SW_ISSUE(j);

  c_lds[t & 63] = bf16_bits_to_f32(cval) * bf16_bits_to_f32(tsv);  // repeated lanes store the same value
  if (LORA) {
    // L[m, r] = sum of the parts in order (zero outside M x R), as bf16 hi + lo
    float sum = 0.0f;
#pragma unroll
    for (int p = 0; p < SS_MAXPARTS; ++p) sum += p < parts ? lv[p] : 0.0f;
    sum = (lm < M && lr < R) ? sum : 0.0f;
    const uint32_t hb = f32_to_bf16_bits(sum);
    const uint32_t lb = f32_to_bf16_bits(sum - bf16_bits_to_f32(hb));  // exact remainder, rounded
    const bool staged = t < 16 * RP;
    *(staged ? l_hi + lm * SW_RS + lr : reinterpret_cast<uint16_t*>(smem + SW_TRASH)) = (uint16_t)hb;
    *(staged ? l_lo + lm * SW_RS + lr : reinterpret_cast<uint16_t*>(smem + SW_TRASH + 2)) = (uint16_t)lb;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SW_WAVES;
      p_lds[(i / RPP) * SW_RS + i % RPP] = (i % RPP) < R ? (uint16_t)pval[u] : (uint16_t)0;
    }
  }

  float4_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = float4_t{0.f, 0.f, 0.f, 0.f};
  const int kb = 16 * wave + 4 * kg;   // byte of the lane's 8 codes within a chunk row
  const int g = 2 * wave + (kg >> 1);  // their 16-group within the chunk
  // this thread's staging targets and the lane's compute operands, in slot 0
  uint8_t* const wdst = smem + SW_W + (t >> 4) * SS_ROW + 16 * (t & 15);
  uint8_t* const adst = smem + SW_A + (t >> 6) * SS_ROW + 4 * (t & 63);
  uint8_t* const sdst = smem + SW_S + (t >> 5) * SW_SSTR * 4 + 8 * (t & 31);
  uint8_t* const asdst = smem + SW_AS + (t & 511) * 4;
  const uint8_t* const a_op = smem + SW_A + r16 * SS_ROW + kb;
  const uint8_t* const as_op = smem + SW_AS + (g * 16 + r16) * 4;
  const uint8_t* const w_op = smem + SW_W + r16 * SS_ROW + kb;
  const uint8_t* const ws_op = smem + SW_S + (g * SW_SSTR + r16) * 4;
#pragma unroll
  for (int i = 0; i < SS_MAXC; ++i) {
    if (i + SW_AHEAD < SS_MAXC) W4A4_SW_ISSUE(i + SW_AHEAD);
    // every chunk is staged, also past the last one, so the loads stay where they were issued
    const int so = (i & 1) * SW_SLOT;
    *reinterpret_cast<u32x4_t*>(wdst + so) = wr[i];
    *reinterpret_cast<uint32_t*>(adst + so) = ar[i];
    const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(sr[i], false);  // the two wscales, exact
    *reinterpret_cast<u32x2_t*>(sdst + so) = u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sf[0], sf[0])),
                                                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(sf[1], sf[1]))};
    *reinterpret_cast<uint32_t*>(asdst + so) = e4m3_dup_h2bits(asr[i]);  // both halves of the workgroup agree
    lds_barrier();  // also: every wave is done with the chunk this slot held two steps ago
    if (!FULL && i >= nc) continue;  // workgroup-uniform
    const uint32_t a4 = *reinterpret_cast<const uint32_t*>(a_op + so);
    const uint32_t as2 = *reinterpret_cast<const uint32_t*>(as_op + so);
    const half8_t av = decode8(a4, __builtin_bit_cast(half2_t, as2));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t w4 = *reinterpret_cast<const uint32_t*>(w_op + so + 16 * b * SS_ROW);
      const uint32_t ws2 = *reinterpret_cast<const uint32_t*>(ws_op + so + 16 * b * 4);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(w4, __builtin_bit_cast(half2_t, ws2)), av, acc[b], 0, 0,
                                                      0);
    }
  }
#undef W4A4_SW_ISSUE
  lds_barrier();  // the slots are free: the reduction reuses them

  // partials -> LDS: lane holds m = lane % 16, n = 16b + 4kg + e; rows 16 * 16 .. hold the
  // rank-R term (waves 0..3, one 16-column block each)
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    *reinterpret_cast<float4_t*>(red + (wave * 16 + r16) * SW_RED + 16 * b + 4 * kg) = acc[b];
  if (LORA && wave < 4) {
    float4_t la = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r0 = 0; r0 < RP; r0 += 32) {
      const bf16x8_t pv = *reinterpret_cast<const bf16x8_t*>(p_lds + (16 * wave + r16) * SW_RS + r0 + 8 * kg);
      const bf16x8_t lh = *reinterpret_cast<const bf16x8_t*>(l_hi + r16 * SW_RS + r0 + 8 * kg);
      const bf16x8_t ll = *reinterpret_cast<const bf16x8_t*>(l_lo + r16 * SW_RS + r0 + 8 * kg);
      la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv, lh, la, 0, 0, 0);
      la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv, ll, la, 0, 0, 0);
    }
    *reinterpret_cast<float4_t*>(red + (SW_WAVES * 16 + r16) * SW_RED + 16 * wave + 4 * kg) = la;
  }
  lds_barrier();
  const int m = t >> 6, n = t & 63;
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < SW_WAVES; ++w) s += red[(w * 16 + m) * SW_RED + n];
  float v = s * c_lds[n];
  if (LORA) v += red[(SW_WAVES * 16 + m) * SW_RED + n];
  if (bias != nullptr) v += bf16_bits_to_f32(bias[min(n0 + n, N - 1)]);
  if (m < M && n0 + n < N) y[(size_t)m * N + n0 + n] = (uint16_t)f32_to_bf16_bits(v);
}

// ---- MXFP4 wide variant (M <= 16, K <= 5120 a multiple of 512) ------------------------------
// The wide kernel's streaming with the MX formats (rotate notes, section 3.3: FP-Quant mxfp4): one
// E8M0 scale per 32 K-columns, activation scales (K/32, ms) with ms = M rounded up to 4, weight
// scales (K/32, N).  Per chunk of 512 K-columns thread t loads 16 bytes of weight row t / 16, 4
// bytes of activation row t / 64, the wscales byte of block row t / 64 and column t % 64, and
// (t < 256) the ascales byte of block row t / 16 and row t % 16.  The product runs on
// v_mfma_scale_f32_16x16x128_f8f6f4, which takes the packed E2M1 codes and the E8M0 bytes
// directly: wave w multiplies weight block w % 4 (16 rows) by the 16 activation rows over the
// chunk's K-columns 128 (w / 4) .. +128, lane (i = lane % 16, kq = lane / 16) supplying 16 code
// bytes (32 columns, one scale block) of weight row 16 (w % 4) + i and of activation row i, and
// the two blocks' scale bytes.  The four waves of each weight block meet in LDS in a fixed order;
// the epilogue is the nvfp4 wide kernel's.
constexpr int SX_W = 0;                              // slot: weight rows (SS_ROW bytes each)
constexpr int SX_A = SX_W + SW_BN * SS_ROW;          //       activation rows
constexpr int SX_S = SX_A + 16 * SS_ROW;             //       wscales [16 blocks][64 columns]
constexpr int SX_AS = SX_S + 16 * SW_BN;             //       ascales [16 blocks][16 rows]
constexpr int SX_SLOT = SX_AS + 16 * 16;
constexpr int SX_REDB = (4 + 1) * 16 * SW_RED * 4;   // four K-step partials and the rank-R term
constexpr int SX_EPI = 2 * SX_SLOT > SX_REDB ? 2 * SX_SLOT : SX_REDB;
constexpr int SX_LHI = SX_EPI;
constexpr int SX_LLO = SX_LHI + 16 * SW_RS * 2;
constexpr int SX_P = SX_LLO + 16 * SW_RS * 2;
constexpr int SX_C = SX_P + SW_BN * SW_RS * 2;
constexpr int SX_TRASH = SX_C + SW_BN * 4;
constexpr int SX_LDS = SX_TRASH + 16;
static_assert(SX_LDS <= 160 * 1024, "LDS of one CU");

template <bool LORA, int RP, bool FULL>
__global__ __launch_bounds__(64 * SW_WAVES) void gemm_skinny_mx_kernel(
    const uint8_t* __restrict__ qa, const uint8_t* __restrict__ sa, const float* __restrict__ lora, int parts,
    const uint8_t* __restrict__ qw, const uint8_t* __restrict__ sw, const uint16_t* __restrict__ pu,
    const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias, int M,
    int N, int K, int R, int ms, uint16_t* __restrict__ y) {
  static_assert(!LORA || RP == 32 || RP == 64, "rank padded to one or two MFMA steps");
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint8_t smem[SX_LDS];
  uint16_t* l_hi = reinterpret_cast<uint16_t*>(smem + SX_LHI);
  uint16_t* l_lo = reinterpret_cast<uint16_t*>(smem + SX_LLO);
  uint16_t* p_lds = reinterpret_cast<uint16_t*>(smem + SX_P);
  float* c_lds = reinterpret_cast<float*>(smem + SX_C);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int blk = wave & 3, ks = wave >> 2;  // the wave's weight block and K-step within a chunk
  const int n0 = xcd_tile(blockIdx.x, gridDim.x) * SW_BN;
  const int kbytes = K / 2;
  const int nc = FULL ? SS_MAXC : kbytes / SS_CH;  // 1 .. SS_MAXC

  // ---- epilogue operands first: the oldest loads, complete before the first chunk is used ----
  constexpr int RPP = RP > 0 ? RP : 1;
  constexpr int PPT = LORA ? SW_BN * RP / (64 * SW_WAVES) : 1;
  const uint32_t cval = wcs[min(n0 + (t & 63), N - 1)];
  const uint32_t tsv = wts[0];
  const int lm = t / RPP, lr = t % RPP;  // the (m, r) element of L this thread stages
  float lv[SS_MAXPARTS];
  uint32_t pval[PPT];
  if (LORA) {
    const int at = min(min(lm, M - 1) * R + min(lr, R - 1), M * R - 1);
#pragma unroll
    for (int p = 0; p < SS_MAXPARTS; ++p) lv[p] = lora[(size_t)min(p, parts - 1) * M * R + at];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SW_WAVES;
      pval[u] = pu[(size_t)min(n0 + i / RPP, N - 1) * R + min(i % RPP, R - 1)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  const uint8_t* wsrc = qw + (size_t)min(n0 + (t >> 4), N - 1) * kbytes + 16 * (t & 15);
  const uint8_t* asrc = qa + (size_t)min(t >> 6, M - 1) * kbytes + 4 * (t & 63);
  const uint32_t soff = (uint32_t)((t >> 6) * N + min(n0 + (t & 63), N - 1));       // within a chunk's blocks
  const uint32_t asoff = (uint32_t)((((t & 255) >> 4) * ms) + min(t & 15, M - 1));
  u32x4_t wr[SS_MAXC];
  uint32_t ar[SS_MAXC], sr[SS_MAXC], asr[SS_MAXC];
#define W4A4_SX_ISSUE(j)                                                              \
  do {                                                                                \
    const int c_ = FULL ? (j) : min((j), nc - 1);                                     \
    wr[(j)] = *reinterpret_cast<const u32x4_t*>(wsrc + c_ * SS_CH);                   \
    ar[(j)] = *reinterpret_cast<const uint32_t*>(asrc + c_ * SS_CH);                  \
    sr[(j)] = (sw + (size_t)c_ * 16 * N)[soff];                                       \
    asr[(j)] = (sa + (size_t)c_ * 16 * ms)[asoff];                                    \
    __builtin_amdgcn_sched_barrier(0);                                                \
  } while (0)
#pragma unroll
  for (int j = 0; j < SW_AHEAD; ++j) W4A4_SX_ISSUE(j);

  c_lds[t & 63] = bf16_bits_to_f32(cval) * bf16_bits_to_f32(tsv);  // repeated lanes store the same value
  if (LORA) {
    // L[m, r] = sum of the parts in order (zero outside M x R), as bf16 hi + lo
    float sum = 0.0f;
#pragma unroll
    for (int p = 0; p < SS_MAXPARTS; ++p) sum += p < parts ? lv[p] : 0.0f;
    sum = (lm < M && lr < R) ? sum : 0.0f;
    const uint32_t hb = f32_to_bf16_bits(sum);
    const uint32_t lb = f32_to_bf16_bits(sum - bf16_bits_to_f32(hb));  // exact remainder, rounded
    const bool staged = t < 16 * RP;
    *(staged ? l_hi + lm * SW_RS + lr : reinterpret_cast<uint16_t*>(smem + SX_TRASH)) = (uint16_t)hb;
    *(staged ? l_lo + lm * SW_RS + lr : reinterpret_cast<uint16_t*>(smem + SX_TRASH + 2)) = (uint16_t)lb;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = t + u * 64 * SW_WAVES;
      p_lds[(i / RPP) * SW_RS + i % RPP] = (i % RPP) < R ? (uint16_t)pval[u] : (uint16_t)0;
    }
  }

  float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
  const int kb = 64 * ks + 16 * kq;  // byte of the lane's 32 codes within a chunk row
  const int sb = 4 * ks + kq;        // their scale block within the chunk
  uint8_t* const wdst = smem + SX_W + (t >> 4) * SS_ROW + 16 * (t & 15);
  uint8_t* const adst = smem + SX_A + (t >> 6) * SS_ROW + 4 * (t & 63);
  uint8_t* const sdst = smem + SX_S + t;                 // [block t / 64][column t % 64]
  uint8_t* const asdst = smem + SX_AS + (t & 255);       // [block][row]
  const uint8_t* const w_op = smem + SX_W + (16 * blk + r16) * SS_ROW + kb;
  const uint8_t* const a_op = smem + SX_A + r16 * SS_ROW + kb;
  const uint8_t* const ws_op = smem + SX_S + sb * SW_BN + 16 * blk + r16;
  const uint8_t* const as_op = smem + SX_AS + sb * 16 + r16;
#pragma unroll
  for (int i = 0; i < SS_MAXC; ++i) {
    if (i + SW_AHEAD < SS_MAXC) W4A4_SX_ISSUE(i + SW_AHEAD);
    // every chunk is staged, also past the last one, so the loads stay where they were issued
    const int so = (i & 1) * SX_SLOT;
    *reinterpret_cast<u32x4_t*>(wdst + so) = wr[i];
    *reinterpret_cast<uint32_t*>(adst + so) = ar[i];
    sdst[so] = (uint8_t)sr[i];
    if (t < 256) asdst[so] = (uint8_t)asr[i];
    lds_barrier();  // also: every wave is done with the chunk this slot held two steps ago
    if (!FULL && i >= nc) continue;  // workgroup-uniform
    const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(w_op + so);
    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(a_op + so);
    const int wsc = ws_op[so], asc = as_op[so];
    // FP4 operands occupy the first four registers of the instruction's eight
    const i32x4_t w4 = __builtin_bit_cast(i32x4_t, wv), a4 = __builtin_bit_cast(i32x4_t, av);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_shufflevector(w4, w4, 0, 1, 2, 3, -1, -1, -1, -1),
                                                          __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1), acc,
                                                          4, 4, 0, wsc, 0, asc);
  }
#undef W4A4_SX_ISSUE
  lds_barrier();  // the slots are free: the reduction reuses them

  // partials -> LDS: lane holds m = lane % 16, n = 16 blk + 4 kq + e of K-step ks; rows 4 * 16 ..
  // hold the rank-R term (waves 0..3, one 16-column block each)
  float* red = reinterpret_cast<float*>(smem);
  *reinterpret_cast<float4_t*>(red + (ks * 16 + r16) * SW_RED + 16 * blk + 4 * kq) = acc;
  if (LORA && wave < 4) {
    float4_t la = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r0 = 0; r0 < RP; r0 += 32) {
      const bf16x8_t pv = *reinterpret_cast<const bf16x8_t*>(p_lds + (16 * wave + r16) * SW_RS + r0 + 8 * kq);
      const bf16x8_t lh = *reinterpret_cast<const bf16x8_t*>(l_hi + r16 * SW_RS + r0 + 8 * kq);
      const bf16x8_t ll = *reinterpret_cast<const bf16x8_t*>(l_lo + r16 * SW_RS + r0 + 8 * kq);
      la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv, lh, la, 0, 0, 0);
      la = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pv, ll, la, 0, 0, 0);
    }
    *reinterpret_cast<float4_t*>(red + (4 * 16 + r16) * SW_RED + 16 * wave + 4 * kq) = la;
  }
  lds_barrier();
  const int m = t >> 6, n = t & 63;
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) s += red[(w * 16 + m) * SW_RED + n];
  float v = s * c_lds[n];
  if (LORA) v += red[(4 * 16 + m) * SW_RED + n];
  if (bias != nullptr) v += bf16_bits_to_f32(bias[min(n0 + n, N - 1)]);
  if (m < M && n0 + n < N) y[(size_t)m * N + n0 + n] = (uint16_t)f32_to_bf16_bits(v);
}

template <int MB, bool VEC16>
hipError_t launch_mb(bool lora_on, hipStream_t st, const uint8_t* qa, const uint8_t* sa, const float* lora, int parts,
                     const uint8_t* qw, const uint8_t* sw, const uint16_t* pu, const uint16_t* wcs, const uint16_t* wts,
                     const uint16_t* bias, int M, int N, int K, int R, uint16_t* y) {
  dim3 grid((unsigned)((N + SK_BN - 1) / SK_BN)), block(64 * SK_WAVES);
  if (lora_on)
    gemm_skinny_kernel<MB, VEC16, true><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  else
    gemm_skinny_kernel<MB, VEC16, false><<<grid, block, 0, st>>>(qa, sa, lora, parts, qw, sw, pu, wcs, wts, bias, M, N, K, R, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const void* qact, const void* ascales, const float* lora, int lora_parts,
                              const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                              const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                              void* y, hipStream_t stream) {
  auto qa = static_cast<const uint8_t*>(qact);
  auto sa = static_cast<const uint8_t*>(ascales);
  auto qw = static_cast<const uint8_t*>(qweight);
  auto sw = static_cast<const uint8_t*>(wscales);
  auto pu = static_cast<const uint16_t*>(proj_up);
  auto wc = static_cast<const uint16_t*>(wcscales);
  auto wt = static_cast<const uint16_t*>(wtscale);
  auto bs = static_cast<const uint16_t*>(bias);
  auto yp = static_cast<uint16_t*>(y);
  const bool vec16 = (K % 32) == 0, lo = R > 0;
  const int m = (int)M, n = (int)N, k = (int)K, r = (int)R;
  // the W4A4_SKINNY_PATH=wide|stream|regs test hook picks a variant; by default the wide kernel
  // serves more than 8192 columns, where the 32-row variants would need two workgroups per CU
  const char* path = test_hook("W4A4_SKINNY_PATH");
  const bool streamed = M <= 16 && (M % 4) == 0 && (K % (2 * SS_CH)) == 0 && K <= 2 * SS_CH * SS_MAXC &&
                        (N % 4) == 0 && ((reinterpret_cast<uintptr_t>(sa) & 3) == 0) &&
                        lora_parts <= SS_MAXPARTS &&
                        ((reinterpret_cast<uintptr_t>(sw) | reinterpret_cast<uintptr_t>(qa)) & 7) == 0 &&
                        !(path && !strcmp(path, "regs"));
  const bool wide = M <= 16 && (K % (2 * SS_CH)) == 0 && K <= 2 * SS_CH * SS_MAXC && (N % 2) == 0 &&
                    ((reinterpret_cast<uintptr_t>(sw) & 1) == 0) && lora_parts <= SS_MAXPARTS &&
                    (path ? !strcmp(path, "wide") : N > 8192);
  if (wide) {
    dim3 grid((unsigned)((N + SW_BN - 1) / SW_BN)), block(64 * SW_WAVES);
    const bool full = K == 2 * SS_CH * SS_MAXC;
#define W4A4_SW_LAUNCH(LO, RP, FU) \
  gemm_skinny_wide_kernel<LO, RP, FU><<<grid, block, 0, stream>>>(qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp)
    if (!lo) {
      if (full) W4A4_SW_LAUNCH(false, 0, true); else W4A4_SW_LAUNCH(false, 0, false);
    } else if (r <= 32) {
      if (full) W4A4_SW_LAUNCH(true, 32, true); else W4A4_SW_LAUNCH(true, 32, false);
    } else {
      if (full) W4A4_SW_LAUNCH(true, 64, true); else W4A4_SW_LAUNCH(true, 64, false);
    }
#undef W4A4_SW_LAUNCH
    return hipGetLastError();
  }
  if (streamed) {
    dim3 grid((unsigned)((N + SK_BN - 1) / SK_BN)), block(64 * SK_WAVES);
    if (lo)
      gemm_skinny_stream_kernel<true><<<grid, block, 0, stream>>>(qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
    else
      gemm_skinny_stream_kernel<false><<<grid, block, 0, stream>>>(qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
    return hipGetLastError();
  }
  if (M <= 16) {
    if (vec16) return launch_mb<1, true>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
    return launch_mb<1, false>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
  }
  if (vec16) return launch_mb<2, true>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
  return launch_mb<2, false>(lo, stream, qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, yp);
}

bool skinny_mx_supported(int64_t M, int64_t K, int64_t R, int lora_parts) {
  return M >= 1 && M <= 16 && K % (2 * SS_CH) == 0 && K <= 2 * SS_CH * SS_MAXC && R <= 64 && lora_parts >= 1 &&
         lora_parts <= SS_MAXPARTS;
}

hipError_t launch_gemm_skinny_mx(const void* qact, const void* ascales, const float* lora, int lora_parts,
                                 const void* qweight, const void* wscales, const void* proj_up, const void* wcscales,
                                 const void* wtscale, const void* bias, int64_t M, int64_t N, int64_t K, int64_t R,
                                 int64_t ms, void* y, hipStream_t stream) {
  if (!skinny_mx_supported(M, K, R, lora_parts)) return hipErrorInvalidValue;
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
  dim3 grid((unsigned)((N + SW_BN - 1) / SW_BN)), block(64 * SW_WAVES);
  const bool full = K == 2 * SS_CH * SS_MAXC;
#define W4A4_SX_LAUNCH(LO, RP, FU) \
  gemm_skinny_mx_kernel<LO, RP, FU><<<grid, block, 0, stream>>>(qa, sa, lora, lora_parts, qw, sw, pu, wc, wt, bs, m, n, k, r, s, yp)
  if (R == 0) {
    if (full) W4A4_SX_LAUNCH(false, 0, true); else W4A4_SX_LAUNCH(false, 0, false);
  } else if (R <= 32) {
    if (full) W4A4_SX_LAUNCH(true, 32, true); else W4A4_SX_LAUNCH(true, 32, false);
  } else {
    if (full) W4A4_SX_LAUNCH(true, 64, true); else W4A4_SX_LAUNCH(true, 64, false);
  }
#undef W4A4_SX_LAUNCH
  return hipGetLastError();
}

}  // namespace w4a4
