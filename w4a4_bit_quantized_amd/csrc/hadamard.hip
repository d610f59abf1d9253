// Standalone block Hadamard transform (gfx950).
//
// Rotate notes, section 3.1 (the Hadacore kernel behind hadacore_transform(x, inplace): a
// Sylvester Hadamard transform applied through its recursion, O(n log n), no stored matrix,
// symmetric and therefore its own inverse, optionally in place; section 3.2 applies it per
// head_dim block and to column partitions of a linear layer's output) and sections 2.1-2.2
// (the Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]], normalised by 1/sqrt(n)).
//
// For every row r and every B-block of the chosen columns,
//   y[r, block] = store( f32(1/sqrt(B)) * FWHT_B(f32(x[r, block])) )
// with butterfly spans 1, 2, ..., B/2 in that order, each pair (a, b) -> (a + b, a - b) in
// float32, then one multiply, then one round-to-nearest-even to the storage type -- the same
// operations in the same order as the rotation fused into the quantizer.
//
// Work decomposition.  A wave owns a unit of U = max(B, 512) consecutive columns of one row:
// lane l holds columns 512 g + 8 l .. + 8 of the unit for g < G = U / 512, loaded as 16-byte
// vectors.  Spans 1, 2, 4 stay inside a lane, spans 8 .. 256 pair lane l with l ^ (span / 8)
// (DPP, ds_swizzle or ds_bpermute: lane_xor), spans of 512 and more pair register groups g and
// g ^ (span / 512) inside the lane.  A unit past the end of a row leaves its trailing lanes idle
// (their blocks do not exist: every block lies inside one unit).  Each wave reads its whole unit
// before writing any of it, so the transform may run in place.

#include "device_common.h"
#include "launch.h"

namespace w4a4 {

namespace {

constexpr int FW_WAVES = 4;

// Storage types: 0 bf16, 1 f16, 2 f32.
template <int DT>
__device__ __forceinline__ float widen(const void* base, int64_t i) {
  if constexpr (DT == 0) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  if constexpr (DT == 1) return (float)static_cast<const _Float16*>(base)[i];
  return static_cast<const float*>(base)[i];
}

template <int DT>
__device__ __forceinline__ void narrow(void* base, int64_t i, float v) {
  if constexpr (DT == 0) static_cast<uint16_t*>(base)[i] = (uint16_t)f32_to_bf16_bits(v);
  else if constexpr (DT == 1) static_cast<_Float16*>(base)[i] = (_Float16)v;  // round to nearest even
  else static_cast<float*>(base)[i] = v;
}

// Eight consecutive elements at element offset i (16-byte aligned for bf16 / f16, 32 bytes of
// f32 as two 16-byte loads).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&v)[8]) {
  if constexpr (DT == 2) {
    const float4_t a = *reinterpret_cast<const float4_t*>(static_cast<const float*>(base) + i);
    const float4_t b = *reinterpret_cast<const float4_t*>(static_cast<const float*>(base) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
  } else if constexpr (DT == 1) {
    const half8_t h = *reinterpret_cast<const half8_t*>(static_cast<const _Float16*>(base) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)h[e];
  } else {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t i, const float (&v)[8]) {
  if constexpr (DT == 2) {
    *reinterpret_cast<float4_t*>(static_cast<float*>(base) + i) = float4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<float4_t*>(static_cast<float*>(base) + i + 4) = float4_t{v[4], v[5], v[6], v[7]};
  } else if constexpr (DT == 1) {
    half8_t h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)v[e];  // round to nearest even
    *reinterpret_cast<half8_t*>(static_cast<_Float16*>(base) + i) = h;
  } else {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = f32_to_bf16_bits(v[2 * e]) | (f32_to_bf16_bits(v[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(base) + i) = w;
  }
}

// The value of lane l ^ d (d a power of two below 64, known at compile time after unrolling):
// DPP quad permutes for 1 and 2, ds_swizzle in bit-mask mode (within 32 lanes) for 4, 8 and 16,
// ds_bpermute for 32.
__device__ __forceinline__ float lane_xor(float v, int d) {
  const int b = __float_as_int(v);
  switch (d) {
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    case 4: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (4 << 10)));
    case 8: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (8 << 10)));
    case 16: return __int_as_float(__builtin_amdgcn_ds_swizzle(b, 0x1F | (16 << 10)));
    default: return __shfl_xor(v, 32);
  }
}

// LOG2B = log2(B); VEC: 16-byte vector loads and stores (pointers, row strides and the column
// count allow them), else one element at a time.
template <int DT, int LOG2B, bool VEC>
__global__ __launch_bounds__(64 * FW_WAVES) void fwht_kernel(const void* x, int64_t ldx, void* y, int64_t ldy,
                                                             int64_t units, int upr, int cols, float norm) {
  constexpr int B = 1 << LOG2B;
  constexpr int G = B > 512 ? B / 512 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * FW_WAVES;
  for (int64_t u = (int64_t)blockIdx.x * FW_WAVES + (threadIdx.x >> 6); u < units; u += stride) {
    const int64_t r = u / upr;
    const int c0 = (int)(u - r * upr) * (512 * G);
    const void* xr = static_cast<const uint8_t*>(x) + r * ldx * (DT == 2 ? 4 : 2);
    void* yr = static_cast<uint8_t*>(y) + r * ldy * (DT == 2 ? 4 : 2);
    float v[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int col = c0 + 512 * g + 8 * lane;
      if (VEC) {
        if (col < cols) {
          load8<DT>(xr, col, v[g]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[g][i] = 0.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[g][i] = col + i < cols ? widen<DT>(xr, col + i) : 0.0f;
      }
    }
    // spans 1, 2, 4: inside the lane's 8 columns
#pragma unroll
    for (int s = 1; s < 8 && s < B; s *= 2)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & s) == 0) {
            const float a = v[g][i], b = v[g][i + s];
            v[g][i] = a + b;
            v[g][i + s] = a - b;
          }
    // spans 8 .. 256: lane l with lane l ^ (span / 8); the lower lane keeps a + b, the upper a - b
#pragma unroll
    for (int s = 8; s < 512 && s < B; s *= 2) {
      const int d = s / 8;
      const bool upper = (lane & d) != 0;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = lane_xor(v[g][i], d);
          v[g][i] = upper ? p - v[g][i] : v[g][i] + p;
        }
    }
    // spans 512 and more: register groups g and g ^ (span / 512)
#pragma unroll
    for (int s = 512; s < B; s *= 2) {
      const int dg = s / 512;
#pragma unroll
      for (int g = 0; g < G; ++g)
        if ((g & dg) == 0)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float a = v[g][i], b = v[g + dg][i];
            v[g][i] = a + b;
            v[g + dg][i] = a - b;
          }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) v[g][i] *= norm;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int col = c0 + 512 * g + 8 * lane;
      if (VEC) {
        if (col < cols) store8<DT>(yr, col, v[g]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (col + i < cols) narrow<DT>(yr, col + i, v[g][i]);
      }
    }
  }
}

template <int DT, int LOG2B>
hipError_t launch_fwht_b(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols, bool vec,
                         float norm, hipStream_t stream) {
  constexpr int U = (1 << LOG2B) > 512 ? (1 << LOG2B) : 512;
  const int upr = (int)((cols + U - 1) / U);
  const int64_t units = rows * upr;
  const int64_t wgs = (units + FW_WAVES - 1) / FW_WAVES;
  const dim3 grid((unsigned)(wgs < 8192 ? wgs : 8192));
  if (vec)
    fwht_kernel<DT, LOG2B, true><<<grid, 64 * FW_WAVES, 0, stream>>>(x, ldx, y, ldy, units, upr, (int)cols, norm);
  else
    fwht_kernel<DT, LOG2B, false><<<grid, 64 * FW_WAVES, 0, stream>>>(x, ldx, y, ldy, units, upr, (int)cols, norm);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_fwht_dt(int log2b, const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                          bool vec, float norm, hipStream_t st) {
  switch (log2b) {
    case 1: return launch_fwht_b<DT, 1>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 2: return launch_fwht_b<DT, 2>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 3: return launch_fwht_b<DT, 3>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 4: return launch_fwht_b<DT, 4>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 5: return launch_fwht_b<DT, 5>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 6: return launch_fwht_b<DT, 6>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 7: return launch_fwht_b<DT, 7>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 8: return launch_fwht_b<DT, 8>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 9: return launch_fwht_b<DT, 9>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 10: return launch_fwht_b<DT, 10>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 11: return launch_fwht_b<DT, 11>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    case 12: return launch_fwht_b<DT, 12>(x, ldx, y, ldy, rows, cols, vec, norm, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_hadamard(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols, int block,
                           int dtype, float norm, hipStream_t stream) {
  int log2b = 0;
  while ((1 << log2b) < block) ++log2b;
  const int es = dtype == 2 ? 4 : 2;
  const bool vec = (cols % 8) == 0 && ((ldx * es) % 16) == 0 && ((ldy * es) % 16) == 0 &&
                   ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
  switch (dtype) {
    case 0: return launch_fwht_dt<0>(log2b, x, ldx, y, ldy, rows, cols, vec, norm, stream);
    case 1: return launch_fwht_dt<1>(log2b, x, ldx, y, ldy, rows, cols, vec, norm, stream);
    case 2: return launch_fwht_dt<2>(log2b, x, ldx, y, ldy, rows, cols, vec, norm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w4a4
