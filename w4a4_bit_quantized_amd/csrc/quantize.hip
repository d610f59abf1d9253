// Fused activation / weight quantizer for the SVDQuant W4A4 linear (gfx950).
//
// One HBM pass over the input computes, per row and per 16-group along K
// ("SVDQuant W4A4" page, "Checkpoint contract" and "Runtime support"; rotate
// notes sections 2.1-2.2 and 3.3 for the fused rotation):
//   x_s = x / smooth_factor (activations, IEEE float32) or w * smooth_factor (weights, exact)
//   v   = x_s, or x_s @ H_B^T per contiguous B-block (Sylvester butterflies with
//         spans 1, 2, ..., B/2 in that order, then one multiply by f32(1/sqrt(B)))
//   s8  = e4m3(f32(amax|v| / 6)),  code = e2m1(f32(v / e4m3_value(s8))), 0 when s8 == 0
//   lora_act = x_s @ proj_down (activations only; unrotated x_s)
//
// Work decomposition: one workgroup per 16 rows, its waves splitting K into
// contiguous chunks of whole "units" (32 columns, or one Hadamard block when
// B > 32).  Lane l of a wave holds row l % 16 and the 8 consecutive columns
// 8 * (l / 16) .. +8 of each 32-column step, which is exactly the A-operand
// layout of the 16x16x32 bf16 MFMA used for the low-rank down-projection.
// A 16-group spans lanes l and l ^ 16.  Butterfly spans 1..4 stay in a lane,
// spans 8 and 16 cross lanes (xor 16, xor 32), spans 32 and 64 cross steps.
// The down-projection runs on the matrix cores with x_s split into a bf16
// high part and a bf16 low part (x_s = hi + lo to 16 significant bits); the
// per-wave partial sums are reduced across waves in a fixed order through
// LDS, so results are deterministic.
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int QROWS = 16;        // rows per workgroup
constexpr int QMAX_WAVES = 16;   // waves per workgroup (split of K)

template <int HB>
struct Unit {
  static constexpr int COLS = HB > 32 ? HB : 32;  // columns per unit
  static constexpr int STEPS = COLS / 32;         // 32-column steps per unit
};

template <int HB>
__device__ __forceinline__ float hadamard_scale() {
  if (HB == 16) return __uint_as_float(0x3E800000u);   // 1/4
  if (HB == 32) return __uint_as_float(0x3E3504F3u);   // RN(1/sqrt(32))
  if (HB == 64) return __uint_as_float(0x3E000000u);   // 1/8
  return __uint_as_float(0x3DB504F3u);                 // RN(1/sqrt(128))
}

// Butterfly stage across lanes: partner = lane ^ mask.  The lane whose
// column is lower keeps a + b, the upper one a - b (a = lower value).
__device__ __forceinline__ float xlane_butterfly(float mine, int mask, bool lower) {
  float other = __shfl_xor(mine, mask, 64);
  return lower ? (mine + other) : (other - mine);
}

template <int HB, int S>
__device__ __forceinline__ void fwht_unit(float (&v)[S][8], int oct) {
  // spans 1, 2, 4: inside the lane's 8 consecutive columns
#pragma unroll
  for (int h = 1; h < 8 && h < HB; h *= 2) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((i & h) == 0) {
          float a = v[s][i], b = v[s][i + h];
          v[s][i] = a + b;
          v[s][i + h] = a - b;
        }
      }
    }
  }
  if (HB >= 16) {  // span 8: octets 2j and 2j+1 -> lanes xor 16
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[s][i] = xlane_butterfly(v[s][i], 16, (oct & 1) == 0);
  }
  if (HB >= 32) {  // span 16: octets j and j+2 -> lanes xor 32
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[s][i] = xlane_butterfly(v[s][i], 32, (oct & 2) == 0);
  }
  // spans 32, 64: between 32-column steps held by the same lane
#pragma unroll
  for (int hs = 1; hs < S; hs *= 2) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if ((s & hs) == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float a = v[s][i], b = v[s + hs][i];
          v[s][i] = a + b;
          v[s + hs][i] = a - b;
        }
      }
    }
  }
  const float c = hadamard_scale<HB>();
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[s][i] = v[s][i] * c;
}

// Quantize the lane's 8 values (half of one 16-group) and store codes/scale.
__device__ __forceinline__ void quantize_store(const float (&v)[8], bool store, bool store_scale,
                                               uint8_t* __restrict__ qrow, size_t qoff,
                                               uint8_t* __restrict__ scale_ptr) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  const float s = __fdiv_rn(amax, 6.0f);
  const uint32_t s8 = e4m3_encode_nonneg(s);
  const float sd = e4m3_decode(s8);
  uint32_t word = 0u;
  if (sd != 0.0f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = __fdiv_rn(v[2 * j], sd);
      float b = __fdiv_rn(v[2 * j + 1], sd);
      word |= e2m1_pack2(a, b) << (8 * j);
    }
  }
  if (store) *reinterpret_cast<uint32_t*>(qrow + qoff) = word;
  if (store_scale) *scale_ptr = (uint8_t)s8;
}

template <int HB, bool ACT, int RB>
__global__ __launch_bounds__(1024) void quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam, const uint16_t* __restrict__ pd,
    int M, int K, int R, int pd_vec, int units_per_wave, int nunits,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales, float* __restrict__ lora) {
  constexpr int COLS = Unit<HB>::COLS;
  constexpr int S = Unit<HB>::STEPS;
  constexpr int RP = RB * 16;  // padded rank
  // LDS: per-wave proj_down staging (32 x RP bf16) and the cross-wave LoRA reduction.
  __shared__ __attribute__((aligned(16))) uint16_t pd_lds[RB > 0 ? QMAX_WAVES * 32 * RP : 1];
  __shared__ __attribute__((aligned(16))) float red_lds[RB > 0 ? QMAX_WAVES * QROWS * RP : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int row = lane & 15;
  const int oct = lane >> 4;
  const int m = blockIdx.x * QROWS + row;
  const bool row_ok = m < M;
  const size_t qstride = (size_t)K / 2;
  uint8_t* qrow = q + (size_t)(row_ok ? m : 0) * qstride;
  const uint16_t* xrow = x + (size_t)(row_ok ? m : 0) * K;

  float4_t acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int rb = 0; rb < (RB > 0 ? RB : 1); ++rb) acc[rb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // blockIdx.y selects a contiguous part of the units (K split across workgroups for small M;
  // each part writes its own low-rank partial sum at lora + part * M * R)
  const int parts = gridDim.y;
  const int per_part = (nunits + parts - 1) / parts;
  const int p_begin = blockIdx.y * per_part;
  const int p_end = min(p_begin + per_part, nunits);
  const int u_begin = p_begin + wave * units_per_wave;
  const int u_end = min(u_begin + units_per_wave, p_end);
  for (int u = u_begin; u < u_end; ++u) {
    float v[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kk = u * COLS + 32 * s + 8 * oct;
      const bool k_ok = kk < K;
      u32x4_t xr = {0u, 0u, 0u, 0u};
      u32x4_t lr = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // 1.0 pairs
      if (k_ok) {
        lr = *reinterpret_cast<const u32x4_t*>(lam + kk);
        if (row_ok) xr = *reinterpret_cast<const u32x4_t*>(xrow + kk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = __uint_as_float(xr[i] << 16), x1 = __uint_as_float(xr[i] & 0xFFFF0000u);
        float l0 = __uint_as_float(lr[i] << 16), l1 = __uint_as_float(lr[i] & 0xFFFF0000u);
        if (ACT) {
          v[s][2 * i] = __fdiv_rn(x0, l0);
          v[s][2 * i + 1] = __fdiv_rn(x1, l1);
        } else {
          v[s][2 * i] = x0 * l0;  // bf16 * bf16 is exact in float32
          v[s][2 * i + 1] = x1 * l1;
        }
      }
      if (ACT && RB > 0) {
        // --- low-rank down-projection on the unrotated x_s -------------------------
        const int k0 = u * COLS + 32 * s;
        uint16_t* my_pd = pd_lds + wave * 32 * RP;
        wave_lds_sync();
        if (pd_vec) {  // 16-byte aligned rows of 8 consecutive ranks
          for (int e = lane * 8; e < 32 * RP; e += 64 * 8) {
            const int r_ = e / RP, c_ = e % RP;  // 8 consecutive columns of one row
            u32x4_t val = {0u, 0u, 0u, 0u};
            if (k0 + r_ < K && c_ < R) val = *reinterpret_cast<const u32x4_t*>(pd + (size_t)(k0 + r_) * R + c_);
            *reinterpret_cast<u32x4_t*>(my_pd + e) = val;
          }
        } else {
          for (int e = lane; e < 32 * RP; e += 64) {
            const int r_ = e / RP, c_ = e % RP;
            uint16_t val = 0;
            if (k0 + r_ < K && c_ < R) val = pd[(size_t)(k0 + r_) * R + c_];
            my_pd[e] = val;
          }
        }
        wave_lds_sync();
        bf16x8_t hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float f = v[s][i];
          const uint32_t hb = f32_to_bf16_bits(f);
          const float rem = f - bf16_bits_to_f32(hb);  // exact
          hi[i] = bf16_from_bits(hb);
          lo[i] = bf16_from_bits(f32_to_bf16_bits(rem));
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          bf16x8_t b;
#pragma unroll
          for (int i = 0; i < 8; ++i) b[i] = bf16_from_bits(my_pd[(8 * oct + i) * RP + rb * 16 + row]);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[rb], 0, 0, 0);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[rb], 0, 0, 0);
        }
      }
    }
    if (HB > 0) fwht_unit<HB, S>(v, oct);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kk = u * COLS + 32 * s + 8 * oct;
      const bool k_ok = kk < K;
      const bool do_store = k_ok && row_ok;
      uint8_t* sp = scales + (size_t)(kk >> 4) * M + (row_ok ? m : 0);
      quantize_store(v[s], do_store, do_store && (oct & 1) == 0, qrow, (size_t)(kk >> 1), sp);
    }
  }

  if (ACT && RB > 0) {
    // --- deterministic cross-wave reduction of the low-rank partials -------------------
    float* my_red = red_lds + wave * QROWS * RP;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) my_red[(oct * 4 + j) * RP + rb * 16 + row] = acc[rb][j];
    __syncthreads();
    for (int t = threadIdx.x; t < QROWS * R; t += blockDim.x) {
      const int rr = t / R, cc = t % R;
      float sum = 0.0f;
      for (int w = 0; w < nwaves; ++w) sum += red_lds[w * QROWS * RP + rr * RP + cc];
      const int mm = blockIdx.x * QROWS + rr;
      if (mm < M) lora[(size_t)blockIdx.y * M * R + (size_t)mm * R + cc] = sum;
    }
  }
}

template <int HB, bool ACT>
hipError_t launch_rb(int rb, dim3 grid, dim3 block, hipStream_t st, const uint16_t* x, const uint16_t* lam,
                     const uint16_t* pd, int M, int K, int R, int pd_vec, int upw, int nunits, uint8_t* q,
                     uint8_t* sc, float* lora) {
  switch (rb) {
    case 0: quantize_kernel<HB, ACT, 0><<<grid, block, 0, st>>>(x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora); break;
    case 1: quantize_kernel<HB, ACT, 1><<<grid, block, 0, st>>>(x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora); break;
    case 2: quantize_kernel<HB, ACT, 2><<<grid, block, 0, st>>>(x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora); break;
    case 3: quantize_kernel<HB, ACT, 3><<<grid, block, 0, st>>>(x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora); break;
    default: quantize_kernel<HB, ACT, 4><<<grid, block, 0, st>>>(x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora); break;
  }
  return hipGetLastError();
}

template <bool ACT>
hipError_t launch_hb(int hb, int rb, dim3 grid, dim3 block, hipStream_t st, const uint16_t* x,
                     const uint16_t* lam, const uint16_t* pd, int M, int K, int R, int pd_vec, int upw,
                     int nunits, uint8_t* q, uint8_t* sc, float* lora) {
  switch (hb) {
    case 0: return launch_rb<0, ACT>(rb, grid, block, st, x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora);
    case 16: return launch_rb<16, ACT>(rb, grid, block, st, x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora);
    case 32: return launch_rb<32, ACT>(rb, grid, block, st, x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora);
    case 64: return launch_rb<64, ACT>(rb, grid, block, st, x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora);
    default: return launch_rb<128, ACT>(rb, grid, block, st, x, lam, pd, M, K, R, pd_vec, upw, nunits, q, sc, lora);
  }
}

}  // namespace

int quantize_parts(int64_t M, int64_t K) {
  // Small batches split K across workgroups so that enough CUs stream x; the partial
  // low-rank sums are added in a fixed order by the consumer.
  const int64_t n32 = K / 32;
  if (M > SKINNY_MAX_M || n32 < 32) return 1;
  return (int)(n32 / 16 < 8 ? n32 / 16 : 8);
}

hipError_t launch_quantize(bool act, const void* x, const void* lam, const void* pd, int64_t M, int64_t K,
                           int64_t R, int hb, int parts, void* q, void* scales, float* lora, hipStream_t stream) {
  const int cols = hb > 32 ? hb : 32;
  const int nunits = (int)((K + cols - 1) / cols);
  const int per_part = (nunits + parts - 1) / parts;
  int nwaves = per_part < QMAX_WAVES ? per_part : QMAX_WAVES;
  const int upw = (per_part + nwaves - 1) / nwaves;
  nwaves = (per_part + upw - 1) / upw;
  const int rb = act ? (int)((R + 15) / 16) : 0;
  dim3 grid((unsigned)((M + QROWS - 1) / QROWS), (unsigned)parts);
  dim3 block((unsigned)(64 * nwaves));
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* lp = static_cast<const uint16_t*>(lam);
  const uint16_t* pp = static_cast<const uint16_t*>(pd);
  uint8_t* qp = static_cast<uint8_t*>(q);
  uint8_t* sp = static_cast<uint8_t*>(scales);
  const int pd_vec = (R % 8 == 0) && ((reinterpret_cast<uintptr_t>(pd) & 15) == 0);
  if (act)
    return launch_hb<true>(hb, rb, grid, block, stream, xp, lp, pp, (int)M, (int)K, (int)R, pd_vec, upw, nunits, qp,
                           sp, lora);
  return launch_hb<false>(hb, 0, grid, block, stream, xp, lp, pp, (int)M, (int)K, 0, 0, upw, nunits, qp, sp, nullptr);
}

}  // namespace w4a4
