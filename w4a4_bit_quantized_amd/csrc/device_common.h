// Device helpers shared by the libw4a4 kernels (gfx950 / CDNA4).
//
// Format facts used here (OCP FP4/FP8 definitions; the "SVDQuant W4A4" page
// names the formats as FP4 pairs per byte and float8_e4m3fn scales):
//   * E2M1 codes: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
//   * e4m3fn: bias 7, subnormal step 2^-9, largest finite 448 (0x7E).
// gfx950 conversion instructions used, with the behaviour measured on the
// device (exhaustively for the encoder over |x| < 16):
//   * v_cvt_scalef32_pk_fp4_f32 with scale 1.0: round to nearest even on the
//     E2M1 grid, saturating to +-6, sign of zero kept; first operand -> low nibble.
//   * v_cvt_scalef32_pk_f16_fp4: exact E2M1 -> f16, multiplied by 2^exponent(scale)
//     only (the scale's mantissa is ignored), so it is called with scale 1.0 and
//     the e4m3 scale is applied by a separate exact f16 multiply.
//   * v_cvt_pk_f32_fp8: exact OCP e4m3fn -> f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ __bf16 bf16_from_bits(uint32_t b) {
  uint16_t s = (uint16_t)b;
  return __builtin_bit_cast(__bf16, s);
}

// Encode a non-negative float32 scale as float8_e4m3fn: round to nearest
// even, subnormal step 2^-9, saturating every value >= 448 to 0x7E.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float s) {
  if (!(s < 448.0f)) return 0x7Eu;  // also catches +inf (NaN never reaches here: amax ignores it)
  uint32_t u = __float_as_uint(s);
  int e = (int)(u >> 23) - 127;
  if (e < -6) {
    // subnormal range: integer multiple of 2^-9; s * 512 is exact, rintf is RNE
    return (uint32_t)rintf(s * 512.0f);  // 8 == 0x08, the smallest normal
  }
  uint32_t mant = u & 0x7FFFFFu;
  uint32_t keep = mant >> 20;           // top 3 mantissa bits
  uint32_t rest = mant & 0xFFFFFu;      // dropped 20 bits
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  return code + up;                     // a mantissa carry bumps the exponent field
}

// e4m3fn byte -> float32 (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(b, false);
  return f[0];
}

// Two float32 -> one byte of E2M1 codes (a in the low nibble).
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// Eight E2M1 codes (one dword, element i in nibble i) times an f16 scale pair
// -> eight exact f16 values.
__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t scale2) {
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  h0 = h0 * scale2;
  h1 = h1 * scale2;
  h2 = h2 * scale2;
  h3 = h3 * scale2;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// e4m3 byte -> f16 pair {s, s} (exact: every e4m3 value is an f16 normal).
__device__ __forceinline__ uint32_t e4m3_to_h2bits(uint32_t b) {
  _Float16 h = (_Float16)e4m3_decode(b);
  uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
  return hb | (hb << 16);
}

// Two e4m3 bytes (bits 0-15 of w) -> two f16 (exact), packed in one dword.
__device__ __forceinline__ uint32_t e4m3x2_to_h2bits(uint32_t w) {
  float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1]));  // exact: no rounding occurs
  return __builtin_bit_cast(uint32_t, h);
}

// {s, s} from the low (hi == 0) or high half of a packed f16 pair.
__device__ __forceinline__ half2_t scale_pair(uint32_t packed, int hi) {
  half2_t p = __builtin_bit_cast(half2_t, packed);
  return hi ? half2_t{p[1], p[1]} : half2_t{p[0], p[0]};
}

// Order LDS traffic between lanes of one wave (wave-private LDS regions).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace w4a4
