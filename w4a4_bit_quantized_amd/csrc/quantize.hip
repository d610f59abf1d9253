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
// Work decomposition.  A workgroup owns 16 rows (consecutive workgroups go to the 8 XCDs in
// turn, so workgroup b takes row block xcd_block(b): each XCD runs a contiguous range of row
// blocks, and the 16-byte pieces that eight row blocks write into each 128-byte line of the
// (K/16, M) scale rows meet in one L2 instead of eight); its waves split K into
// contiguous runs of units (64 columns, or 128 for B = 128).  A unit is one or
// two 64-column steps.  In a step, lane l holds row l % 16 and the 16
// consecutive columns 16 * (l / 16) .. +16: exactly one quantization group, so
// the group maximum, the scale and the eight code bytes stay inside the lane.
// Butterfly spans 1..8 are in-lane; spans 16 and 32 pair lane l with l ^ 16 and
// l ^ 32 (v_permlane16_swap / v_permlane32_swap on pairs of registers: one
// swap brings both partners' values together, every lane forms a + b and
// a - b, a second swap returns the results); span 64 joins the two steps of a
// 128-column unit.
//
// Division.  Both divisions are correctly rounded without a divide instruction
// per element.  x / lambda uses a two-part reciprocal of lambda = m 2^E (m the
// bf16 mantissa, one of 128 values): rh = RD(1/m) 2^-E and rl = RN((1 - m RD(1/m))
// RD(1/m)) 2^-E, both from a 128-entry table built once per workgroup (the
// residual 1 - m RD(1/m) is exact and >= 0), then per element
//   q = RN(x rh + RN(x rl))   (one multiply and one fused multiply-add).
// rh + rl is within 2^-46 of 1/lambda, and a quotient of two 8-bit mantissas is
// either a float32 or farther than that from every rounding midpoint, so for
// bf16 x with 2^-64 <= |x| < 2^96 (or x = +-0; rl >= 0 keeps the sign of a zero)
// and bf16 lambda in [2^-32, 2^32] this equals RN(x / lambda) bit for bit
// (checked exhaustively over every pair of bf16 mantissas and the exponent
// offsets); units or waves whose inputs fall outside that range take the IEEE
// division instead.  v / sd uses r = RN(1/sd) from a 128-entry table and one
// Markstein correction,
//   q0 = RN(v r),  e = RN(q0 sd - v) (exact, fused),  q = RN(q0 - e r);
// there the E2M1 code of the result equals the code of the IEEE quotient for
// every finite v and every nonzero e4m3 sd reachable from the group maximum
// (checked near every decision point and across all binades); groups whose
// maximum is not finite take the IEEE division.
//
// Low-rank down-projection.  x_s is split into a bf16 high part and a bf16 low
// part (x_s = hi + lo to about 16 significant bits) that feed the 16x16x32 bf16
// MFMA as the A operand: lane (row, quarter q) supplies columns 16q .. 16q+8 of
// its group in one MFMA and 16q+8 .. 16q+16 in the next.  The matching
// proj_down operand is staged per wave in LDS, row-major as in memory, and read
// with the transposing ds_read_b64_tr_b16, which hands each lane four
// consecutive K-rows of one rank column.  Per-wave partial sums are reduced
// across waves in a fixed order through LDS, so results are deterministic.
#include "device_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int QROWS = 16;  // rows per workgroup

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Waves per workgroup, set by the register budget of the variant: 16 (four per SIMD) where a wave
// needs at most 128 VGPRs; 12 (three per SIMD) for the 128-point rotation with rank <= 32 (140-145
// VGPRs: twelve waves hide more latency than eight, sixteen would spill); 8 above rank 32.
constexpr int max_waves(int hb, int rb) { return rb > 2 ? 8 : (hb == 128 && rb > 0) ? 12 : 16; }

template <int HB, bool ACT, int RB>
struct QCfg {
  static constexpr int UC = HB == 128 ? 128 : 64;  // columns per unit
  static constexpr int US = UC / 64;               // 64-column steps per unit
  static constexpr int RP = RB * 16;               // padded rank
  static constexpr int RS = RP + 16;               // LDS row stride of proj_down (u16), 32 bytes of padding
  static constexpr int WAVES = max_waves(HB, RB);  // most waves per workgroup (register budget)
  static constexpr int PD_BYTES = (ACT && RB > 0) ? 64 * RS * 2 : 0;
  static constexpr int LAM_BYTES = ACT ? 3 * UC * 4 : 0;   // lambda, rh, rl of the unit's columns
  static constexpr int WAVE_BYTES = PD_BYTES + LAM_BYTES;
  static constexpr int RED_BYTES = (ACT && RB > 0) ? WAVES * QROWS * RP * 4 : 0;
  static constexpr int BODY_BYTES = WAVES * WAVE_BYTES > RED_BYTES ? WAVES * WAVE_BYTES : RED_BYTES;
  static constexpr int TAB_BYTES = 512 + 1024;       // reciprocals of the e4m3 scales, then (rh, rl) of the bf16 mantissas
  static constexpr int LDS_BYTES = TAB_BYTES + BODY_BYTES;
};

// Row block of workgroup b of G when workgroups are dispatched to the 8 XCDs in turn: XCD x runs
// a contiguous range of blocks (a bijection on [0, G) for any G).
__device__ __forceinline__ int xcd_block(int b, int G) {
  const int q = G / 8, r = G % 8, x = b % 8, l = b / 8;
  return x < r ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;
}

template <int HB>
__device__ __forceinline__ float hadamard_scale() {
  if (HB == 16) return __uint_as_float(0x3E800000u);   // 1/4
  if (HB == 32) return __uint_as_float(0x3E3504F3u);   // RN(1/sqrt(32))
  if (HB == 64) return __uint_as_float(0x3E000000u);   // 1/8
  return __uint_as_float(0x3DB504F3u);                 // RN(1/sqrt(128))
}

// Butterfly between lanes l and l ^ 16 (SWAP32 = false) or l ^ 32 (true) on two
// registers at once.  The lane with the lower column keeps a + b, the other a - b.
template <bool SWAP32>
__device__ __forceinline__ void xlane_pair(float& a, float& b) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  uint32_t p0, p1;
  if (SWAP32) {
    auto s = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
    p0 = s[0]; p1 = s[1];
  } else {
    auto s = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    p0 = s[0]; p1 = s[1];
  }
  // lower lane now holds (a_low, a_high), upper lane (b_low, b_high)
  const float lo = __uint_as_float(p0), hi = __uint_as_float(p1);
  const float sum = lo + hi, dif = lo - hi;
  uint32_t r0, r1;
  if (SWAP32) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(dif), false, false);
    r0 = s[0]; r1 = s[1];
  } else {
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(sum), __float_as_uint(dif), false, false);
    r0 = s[0]; r1 = s[1];
  }
  a = __uint_as_float(r0);
  b = __uint_as_float(r1);
}

template <int HB, int US>
__device__ __forceinline__ void fwht_unit(float (&v)[US][16]) {
  // spans 1, 2, 4, 8: inside the lane's 16 consecutive columns
#pragma unroll
  for (int h = 1; h < 16 && h < HB; h *= 2)
#pragma unroll
    for (int c = 0; c < US; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i & h) == 0) {
          const float a = v[c][i], b = v[c][i + h];
          v[c][i] = a + b;
          v[c][i + h] = a - b;
        }
  if (HB >= 32)  // span 16: lanes l and l ^ 16
#pragma unroll
    for (int c = 0; c < US; ++c)
#pragma unroll
      for (int i = 0; i < 16; i += 2) xlane_pair<false>(v[c][i], v[c][i + 1]);
  if (HB >= 64)  // span 32: lanes l and l ^ 32
#pragma unroll
    for (int c = 0; c < US; ++c)
#pragma unroll
      for (int i = 0; i < 16; i += 2) xlane_pair<true>(v[c][i], v[c][i + 1]);
  if (HB >= 128)  // span 64: the unit's two steps
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float a = v[0][i], b = v[US - 1][i];
      v[0][i] = a + b;
      v[US - 1][i] = a - b;
    }
  const float cb = hadamard_scale<HB>();
#pragma unroll
  for (int c = 0; c < US; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) v[c][i] = v[c][i] * cb;
}

// v / d with the E2M1 code of the IEEE quotient (see the top of the file).
__device__ __forceinline__ float div_markstein(float x, float d, float r) {
  const float q0 = x * r;
  const float e = fmaf(q0, d, -x);
  return fmaf(-e, r, q0);
}

// Eight float32 -> eight E2M1 codes in one dword (element i in nibble i).
__device__ __forceinline__ uint32_t pack8(const float (&t)[8]) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[0], t[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[2], t[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[4], t[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[6], t[7], 1.0f, 3);
}

// Quantize one group (the lane's 16 values): 8 code bytes and the scale byte.
__device__ __forceinline__ void quantize_group(const float (&v)[16], const float* rtab, u32x2_t& codes,
                                               uint32_t& s8) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float s = __fdiv_rn(amax, 6.0f);
  s8 = e4m3_encode_nonneg(s);
  const float sd = e4m3_decode(s8);
  const float rs = rtab[s8];
  uint32_t w[2];
  if (__builtin_amdgcn_ballot_w64(!__builtin_isfinite(amax)) == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = div_markstein(v[8 * h + i], sd, rs);
      w[h] = pack8(t);
    }
  } else {  // some lane's group holds an infinity: IEEE division for the whole wave
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = __fdiv_rn(v[8 * h + i], sd);
      w[h] = pack8(t);
    }
  }
  const bool nz = sd != 0.0f;
  codes = u32x2_t{nz ? w[0] : 0u, nz ? w[1] : 0u};
}

// MXFP4 block of 32 (rotate notes, section 3.3, FP-Quant mxfp4 / abs_max): the lane's 16 values
// and those of lane l ^ 16 (the block's other half).  Scale 2^e with e the least exponent such
// that 2^e >= float32(amax / 6), clamped to the E8M0 range [-127, 127]; the elements are
// multiplied by the exact power of two 2^-e and rounded to E2M1.  Returns the 8 code bytes and
// the E8M0 byte e + 127.  Every lane of the wave must call it (cross-lane exchange).
__device__ __forceinline__ void quantize_block_mx(const float (&v)[16], u32x2_t& codes, uint32_t& e8) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t ab = __float_as_uint(amax);
  const auto sw = __builtin_amdgcn_permlane16_swap(ab, ab, false, false);  // {own, partner} in some order
  amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
  const uint32_t qb = __float_as_uint(__fdiv_rn(amax, 6.0f));
  const uint32_t ex = qb >> 23, mant = qb & 0x7FFFFFu;
  // subnormal q = mant * 2^-149: above 2^-127 exactly when mant > 2^22
  int e = ex == 0 ? (mant > 0x400000u ? -126 : -127) : (int)ex - 127 + (mant != 0u ? 1 : 0);
  e = e > 127 ? 127 : e;
  e8 = (uint32_t)(e + 127);
  const float f = e == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = v[8 * h + i] * f;  // exact (a product below 2^-126 codes to 0 anyway)
    w[h] = pack8(t);
  }
  codes = u32x2_t{w[0], w[1]};
}

// Raw input check for the fast x / lambda: every bf16 in `d` is +-0 or has
// 2^-64 <= |x| < 2^96.  Accumulates packed u16 minima / maxima.
__device__ __forceinline__ void range_acc(uint32_t d, u16x2_t& mn, u16x2_t& mx) {
  const u16x2_t a = __builtin_bit_cast(u16x2_t, d & 0x7FFF7FFFu);
  mn = __builtin_elementwise_min(mn, a - (u16x2_t){1, 1});  // +-0 wraps to 0xFFFF
  mx = __builtin_elementwise_max(mx, a);
}

__device__ __forceinline__ bool range_bad(u16x2_t mn, u16x2_t mx) {
  return (mn[0] < 0x1F7Fu) | (mn[1] < 0x1F7Fu) | (mx[0] >= 0x6F80u) | (mx[1] >= 0x6F80u);
}

// MX selects the MXFP4 blocks (32 columns, E8M0 scales in rows of `ms` bytes: the scale of
// block b of row m is at scales[b * ms + m]; rows M .. ms - 1 receive 0) instead of the
// 16-column e4m3 groups (scales[g * M + m]).
template <int HB, bool ACT, int RB, bool MX>
__global__ __launch_bounds__(64 * max_waves(HB, RB)) void quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam, const uint16_t* __restrict__ pd,
    int M, int K, int R, int units_per_wave, int nunits, int ms,
    uint8_t* __restrict__ q, uint8_t* __restrict__ scales, float* __restrict__ lora) {
  using C = QCfg<HB, ACT, RB>;
  constexpr int US = C::US, UC = C::UC, RP = C::RP, RS = C::RS;
  constexpr bool LORA = ACT && RB > 0;
  constexpr int PDV = LORA ? RP / 8 : 1;  // 16-byte proj_down chunks per lane per step
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  float* rtab = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int row = lane & 15;
  const int qd = lane >> 4;
  const int m0 = xcd_block(blockIdx.x, gridDim.x) * QROWS;
  const int m = m0 + row;
  const bool row_ok = m < M;
  const size_t qstride = (size_t)K / 2;
  // rows past M read row m0 (valid, finite) and never store
  const uint16_t* xrow = x + (size_t)(row_ok ? m : m0) * K;
  uint8_t* qrow = q + (size_t)(row_ok ? m : m0) * qstride;

  float2_t* mtab = reinterpret_cast<float2_t*>(smem + 512);
  uint8_t* wbase = smem + C::TAB_BYTES + wave * C::WAVE_BYTES;
  float* lam_s = reinterpret_cast<float*>(wbase + C::PD_BYTES);
  float* rh_s = lam_s + UC;
  float* rl_s = lam_s + 2 * UC;
  uint16_t* pd_s = reinterpret_cast<uint16_t*>(wbase);

  for (int b = threadIdx.x; b < 128; b += blockDim.x)
    rtab[b] = (b == 0 || b == 127) ? 0.0f : __fdiv_rn(1.0f, e4m3_decode((uint32_t)b));
  if constexpr (ACT) {
    for (int b = threadIdx.x; b < 128; b += blockDim.x) {
      const float mm = __uint_as_float(0x3F800000u | ((uint32_t)b << 16));  // 1 + b/128
      float rh = __fdiv_rn(1.0f, mm);
      if (fmaf(-mm, rh, 1.0f) < 0.0f) rh = __uint_as_float(__float_as_uint(rh) - 1u);  // RD(1/mm)
      mtab[b] = float2_t{rh, fmaf(-mm, rh, 1.0f) * rh};  // the residual is exact and >= 0
    }
  }
  __syncthreads();

  // blockIdx.y selects a contiguous part of the units (K split across workgroups for small M;
  // each part writes its own low-rank partial sum at lora + part * M * R)
  const int parts = gridDim.y;
  const int per_part = (nunits + parts - 1) / parts;
  const int p_begin = blockIdx.y * per_part;
  const int p_end = min(p_begin + per_part, nunits);
  const int u_begin = p_begin + wave * units_per_wave;
  const int u_end = min(u_begin + units_per_wave, p_end);

  float4_t acc[RB > 0 ? RB : 1];
#pragma unroll
  for (int rb = 0; rb < (RB > 0 ? RB : 1); ++rb) acc[rb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // ---- loaders ---------------------------------------------------------------------------
  // x (or w): two 16-byte loads per step; past-K columns read column 0 and are zeroed later.
  auto load_x = [&](int u, u32x4_t (&dst)[US][2]) {
#pragma unroll
    for (int c = 0; c < US; ++c) {
      const int k0 = u * UC + 64 * c + 16 * qd;
      const int kk = k0 < K ? k0 : 0;
      dst[c][0] = *reinterpret_cast<const u32x4_t*>(xrow + kk);
      dst[c][1] = *reinterpret_cast<const u32x4_t*>(xrow + kk + 8);
    }
  };
  // activations: lambda of column u * UC + 64 c + lane (one per lane); weights: the lane's 16 columns
  auto load_lam_act = [&](int u, uint32_t (&dst)[US]) {
#pragma unroll
    for (int c = 0; c < US; ++c) {
      const int k = u * UC + 64 * c + lane;
      dst[c] = k < K ? (uint32_t)lam[k] : 0x3F80u;  // 1.0 past K
    }
  };
  auto load_lam_w = [&](int u, u32x4_t (&dst)[US][2]) {
#pragma unroll
    for (int c = 0; c < US; ++c) {
      const int k0 = u * UC + 64 * c + 16 * qd;
      const int kk = k0 < K ? k0 : 0;
      dst[c][0] = *reinterpret_cast<const u32x4_t*>(lam + kk);
      dst[c][1] = *reinterpret_cast<const u32x4_t*>(lam + kk + 8);
    }
  };
  // proj_down rows k0 .. k0 + 63 (all RP columns, zero past K or R): chunk i of the lane is
  // row (lane + 64 i) / (RP / 8), columns 8 * ((lane + 64 i) % (RP / 8)) .. +8
  auto load_pd = [&](int kstep, u32x4_t (&dst)[PDV]) {
    if constexpr (LORA) {
      const int k0 = kstep * 64;
      const bool full = (R == RP) && (k0 + 64 <= K) && ((R & 7) == 0);
#pragma unroll
      for (int i = 0; i < PDV; ++i) {
        const int ch = lane + 64 * i;
        const int r_ = ch / (RP / 8), c8 = 8 * (ch % (RP / 8));
        const int k = k0 + r_;
        if (full) {
          dst[i] = *reinterpret_cast<const u32x4_t*>(pd + (size_t)k * R + c8);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int c0 = c8 + 2 * e2;
            const uint32_t lo = (k < K && c0 < R) ? (uint32_t)pd[(size_t)k * R + c0] : 0u;
            const uint32_t hi = (k < K && c0 + 1 < R) ? (uint32_t)pd[(size_t)k * R + c0 + 1] : 0u;
            w[e2] = lo | (hi << 16);
          }
          dst[i] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
    }
  };

  u32x4_t xr[US][2];
  u32x4_t lwr[ACT ? 1 : US][2];    // weights: lambda of the lane's columns
  uint32_t lar[ACT ? US : 1];      // activations: lambda of column lane
  u32x4_t pdr[PDV];
  if (u_begin < u_end) {
    load_x(u_begin, xr);
    if constexpr (ACT) load_lam_act(u_begin, lar); else load_lam_w(u_begin, lwr);
    load_pd(u_begin * US, pdr);
  }

  for (int u = u_begin; u < u_end; ++u) {
    // the current unit's raw inputs (the next unit's are fetched into the same registers once
    // these are consumed by the smoothing)
    u32x4_t (&xc)[US][2] = xr;
    const uint32_t (&lac)[ACT ? US : 1] = lar;
    const u32x4_t (&lwc)[ACT ? 1 : US][2] = lwr;
    const bool tail = (u + 1) * UC > K;
    if (tail) {  // zero the columns past K (whole blocks, K being a multiple of the block)
#pragma unroll
      for (int c = 0; c < US; ++c)
        if (u * UC + 64 * c + 16 * qd >= K) {
          xc[c][0] = u32x4_t{0u, 0u, 0u, 0u};
          xc[c][1] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    float v[US][16];
    if constexpr (ACT) {
      // lambda and its two-part reciprocal (rh, rl) of the unit's columns, shared through the
      // wave's LDS; lambda = m 2^E in range scales the mantissa's table entry by 2^-E exactly
      bool lam_ok = true;
#pragma unroll
      for (int c = 0; c < US; ++c) {
        const float lf = bf16_bits_to_f32(lac[c]);
        lam_ok &= (lf >= 0x1p-32f) && (lf <= 0x1p32f);
        const float2_t t = mtab[lac[c] & 0x7Fu];
        const float p2 = __uint_as_float((254u << 23) - (__float_as_uint(lf) & 0x7F800000u));  // 2^-E
        lam_s[64 * c + lane] = lf;
        rh_s[64 * c + lane] = t[0] * p2;
        rl_s[64 * c + lane] = t[1] * p2;
      }
      u16x2_t mn = {0xFFFFu, 0xFFFFu}, mx = {0u, 0u};
#pragma unroll
      for (int c = 0; c < US; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) range_acc(xc[c][h][i], mn, mx);
      const bool fast = __builtin_amdgcn_ballot_w64(!lam_ok || range_bad(mn, mx)) == 0;
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < US; ++c) {
        if (fast) {
          const float* ph = rh_s + 64 * c + 16 * qd;
          const float* pl = rl_s + 64 * c + 16 * qd;
          float hv[16], lw[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4_t a = *reinterpret_cast<const float4_t*>(ph + 4 * i);
            const float4_t b = *reinterpret_cast<const float4_t*>(pl + 4 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) { hv[4 * i + e] = a[e]; lw[4 * i + e] = b[e]; }
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t d = xc[c][h][i];
              const int j = 8 * h + 2 * i;
              const float x0 = __uint_as_float(d << 16), x1 = __uint_as_float(d & 0xFFFF0000u);
              v[c][j] = fmaf(x0, hv[j], x0 * lw[j]);
              v[c][j + 1] = fmaf(x1, hv[j + 1], x1 * lw[j + 1]);
            }
        } else {  // inputs outside the proven range somewhere in the wave: IEEE division
          const float* ls = lam_s + 64 * c + 16 * qd;
          float lv[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4_t a = *reinterpret_cast<const float4_t*>(ls + 4 * i);
#pragma unroll
            for (int e = 0; e < 4; ++e) lv[4 * i + e] = a[e];
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t d = xc[c][h][i];
              const int j = 8 * h + 2 * i;
              v[c][j] = __fdiv_rn(__uint_as_float(d << 16), lv[j]);
              v[c][j + 1] = __fdiv_rn(__uint_as_float(d & 0xFFFF0000u), lv[j + 1]);
            }
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < US; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t d = xc[c][h][i], l = lwc[c][h][i];
            const int j = 8 * h + 2 * i;
            v[c][j] = __uint_as_float(d << 16) * __uint_as_float(l << 16);  // bf16 * bf16: exact
            v[c][j + 1] = __uint_as_float(d & 0xFFFF0000u) * __uint_as_float(l & 0xFFFF0000u);
          }
    }

    if (u + 1 < u_end) {
      load_x(u + 1, xr);
      if constexpr (ACT) load_lam_act(u + 1, lar); else load_lam_w(u + 1, lwr);
    }

    if constexpr (LORA) {
      // ---- low-rank down-projection on the unrotated x_s ------------------------------------
#pragma unroll
      for (int c = 0; c < US; ++c) {
        const int kstep = u * US + c;
        // stage this step's proj_down rows (the wave's previous reads are done: LDS is in order)
#pragma unroll
        for (int i = 0; i < PDV; ++i) {
          const int ch = lane + 64 * i;
          const int r_ = ch / (RP / 8), c8 = 8 * (ch % (RP / 8));
          *reinterpret_cast<u32x4_t*>(pd_s + r_ * RS + c8) = pdr[i];
        }
        if (kstep + 1 < u_end * US) load_pd(kstep + 1, pdr);
        wave_lds_sync();
        bf16x8_t hi[2], lo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float f0 = v[c][8 * h + 2 * j], f1 = v[c][8 * h + 2 * j + 1];
            const bf16x2_t hb = __builtin_convertvector(float2_t{f0, f1}, bf16x2_t);
            const uint32_t hbits = __builtin_bit_cast(uint32_t, hb);
            const float r0 = f0 - __uint_as_float(hbits << 16);  // exact
            const float r1 = f1 - __uint_as_float(hbits & 0xFFFF0000u);
            const bf16x2_t lb = __builtin_convertvector(float2_t{r0, r1}, bf16x2_t);
            hi[h][2 * j] = hb[0]; hi[h][2 * j + 1] = hb[1];
            lo[h][2 * j] = lb[0]; lo[h][2 * j + 1] = lb[1];
          }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // lane (n = lane % 16, quarter qd) receives proj_down[16 qd + 8 h + 4 t + e][16 rb + n]
            const int s = lane & 15;
            const int base = (16 * qd + 8 * h + (s >> 2)) * RS + 16 * rb + 4 * (s & 3);
            typedef __attribute__((address_space(3))) short4_t lds_s4;
            const short4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(pd_s + base));
            const short4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(pd_s + base + 4 * RS));
            const u32x2_t w0 = __builtin_bit_cast(u32x2_t, t0), w1 = __builtin_bit_cast(u32x2_t, t1);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[h], b, acc[rb], 0, 0, 0);
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[h], b, acc[rb], 0, 0, 0);
          }
      }
    }

    if constexpr (HB > 0) fwht_unit<HB, US>(v);

#pragma unroll
    for (int c = 0; c < US; ++c) {
      const int k0 = u * UC + 64 * c + 16 * qd;
      u32x2_t codes;
      uint32_t s8;
      if constexpr (MX) quantize_block_mx(v[c], codes, s8);
      else quantize_group(v[c], rtab, codes, s8);
      if (row_ok && k0 < K) {
        uint32_t* qp = reinterpret_cast<uint32_t*>(qrow + (k0 >> 1));  // 4-byte aligned output
        qp[0] = codes[0];
        qp[1] = codes[1];
        if constexpr (!MX) scales[(size_t)(k0 >> 4) * M + m] = (uint8_t)s8;
      }
      if constexpr (MX) {  // the block's even half stores its scale; padding rows store 0
        if ((qd & 1) == 0 && m < ms && k0 < K) scales[(size_t)(k0 >> 5) * ms + m] = row_ok ? (uint8_t)s8 : (uint8_t)0;
      }
    }
  }

  if constexpr (LORA) {
    // ---- deterministic cross-wave reduction of the low-rank partials ----------------------
    __syncthreads();  // every wave is done with its proj_down staging area
    float* red = reinterpret_cast<float*>(smem + C::TAB_BYTES);
    float* my_red = red + wave * QROWS * RP;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) my_red[(4 * qd + e) * RP + 16 * rb + row] = acc[rb][e];
    __syncthreads();
    for (int t = threadIdx.x; t < QROWS * R; t += blockDim.x) {
      const int rr = t / R, cc = t % R;
      float sum = 0.0f;
      for (int w = 0; w < nwaves; ++w) sum += red[w * QROWS * RP + rr * RP + cc];
      const int mm = m0 + rr;
      if (mm < M) lora[(size_t)blockIdx.y * M * R + (size_t)mm * R + cc] = sum;
    }
  }
}

template <int HB, bool ACT, int RB, bool MX>
hipError_t launch_one(dim3 grid, int nunits, int per_part, int ms, hipStream_t st, const uint16_t* x,
                      const uint16_t* lam, const uint16_t* pd, int M, int K, int R, uint8_t* q, uint8_t* sc,
                      float* lora) {
  using C = QCfg<HB, ACT, RB>;
  int nwaves = per_part < C::WAVES ? per_part : C::WAVES;
  if (nwaves < 1) nwaves = 1;
  const int upw = (per_part + nwaves - 1) / nwaves;
  nwaves = (per_part + upw - 1) / upw;
  if (nwaves < 1) nwaves = 1;
  quantize_kernel<HB, ACT, RB, MX><<<grid, dim3(64 * nwaves), 0, st>>>(x, lam, pd, M, K, R, upw, nunits, ms, q, sc,
                                                                        lora);
  return hipGetLastError();
}

#define W4A4_Q_ARGS grid, nunits, per_part, ms, st, x, lam, pd, M, K, R, q, sc, lora

template <int HB, bool ACT, bool MX>
hipError_t launch_rb(int rb, dim3 grid, int nunits, int per_part, int ms, hipStream_t st, const uint16_t* x,
                     const uint16_t* lam, const uint16_t* pd, int M, int K, int R, uint8_t* q, uint8_t* sc,
                     float* lora) {
  if constexpr (!ACT) {
    return launch_one<HB, false, 0, MX>(W4A4_Q_ARGS);
  } else {
    switch (rb) {
      case 0: return launch_one<HB, true, 0, MX>(W4A4_Q_ARGS);
      case 1: return launch_one<HB, true, 1, MX>(W4A4_Q_ARGS);
      case 2: return launch_one<HB, true, 2, MX>(W4A4_Q_ARGS);
      case 3: return launch_one<HB, true, 3, MX>(W4A4_Q_ARGS);
      default: return launch_one<HB, true, 4, MX>(W4A4_Q_ARGS);
    }
  }
}

template <bool ACT, bool MX>
hipError_t launch_hb(int hb, int rb, dim3 grid, int nunits, int per_part, int ms, hipStream_t st, const uint16_t* x,
                     const uint16_t* lam, const uint16_t* pd, int M, int K, int R, uint8_t* q, uint8_t* sc,
                     float* lora) {
  if constexpr (MX) {  // the MX variant rotates in blocks of 32 or not at all
    switch (hb) {
      case 0: return launch_rb<0, ACT, true>(rb, W4A4_Q_ARGS);
      case 32: return launch_rb<32, ACT, true>(rb, W4A4_Q_ARGS);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (hb) {
      case 0: return launch_rb<0, ACT, false>(rb, W4A4_Q_ARGS);
      case 16: return launch_rb<16, ACT, false>(rb, W4A4_Q_ARGS);
      case 32: return launch_rb<32, ACT, false>(rb, W4A4_Q_ARGS);
      case 64: return launch_rb<64, ACT, false>(rb, W4A4_Q_ARGS);
      default: return launch_rb<128, ACT, false>(rb, W4A4_Q_ARGS);
    }
  }
}

#undef W4A4_Q_ARGS

}  // namespace

hipError_t launch_quantize(bool act, const void* x, const void* lam, const void* pd, int64_t M, int64_t K,
                           int64_t R, int hb, int parts, void* q, void* scales, float* lora, hipStream_t stream,
                           bool mx, int64_t scale_stride) {
  const int uc = hb == 128 ? 128 : 64;
  const int nunits = (int)((K + uc - 1) / uc);
  const int per_part = (nunits + parts - 1) / parts;
  const int rb = act ? (int)((R + 15) / 16) : 0;
  const int ms = mx ? (int)scale_stride : (int)M;
  dim3 grid((unsigned)((M + QROWS - 1) / QROWS), (unsigned)parts);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* lp = static_cast<const uint16_t*>(lam);
  const uint16_t* pp = static_cast<const uint16_t*>(pd);
  uint8_t* qp = static_cast<uint8_t*>(q);
  uint8_t* sp = static_cast<uint8_t*>(scales);
  const int r = act ? (int)R : 0;
  float* lo = act ? lora : nullptr;
  if (act) {
    if (mx) return launch_hb<true, true>(hb, rb, grid, nunits, per_part, ms, stream, xp, lp, pp, (int)M, (int)K, r, qp, sp, lo);
    return launch_hb<true, false>(hb, rb, grid, nunits, per_part, ms, stream, xp, lp, pp, (int)M, (int)K, r, qp, sp, lo);
  }
  if (mx) return launch_hb<false, true>(hb, 0, grid, nunits, per_part, ms, stream, xp, lp, pp, (int)M, (int)K, 0, qp, sp, lo);
  return launch_hb<false, false>(hb, 0, grid, nunits, per_part, ms, stream, xp, lp, pp, (int)M, (int)K, 0, qp, sp, lo);
}

}  // namespace w4a4
