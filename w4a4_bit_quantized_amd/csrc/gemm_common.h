// Pieces shared by the tiled GEMM kernels (gemm.hip, gemm_mx.hip): output-tile order, tile
// geometry, the direct-load issue, the epilogues.  Internal to libw4a4.
#pragma once

#include "device_common.h"

namespace w4a4 {

// Compute units of the current device (cached per device).
int device_cus();

namespace {

constexpr int BK = 128;            // K columns per stage (8 groups of 16)
constexpr int CODE_STRIDE = 80;    // LDS bytes per code row: 64 data + 16 pad (conflict-free b128 reads)

// Output tile (tm, tn) of workgroup b among G tiles of a tiles_m x tiles_n grid.  Workgroups are
// dispatched to the 8 XCDs in turn; each XCD takes a contiguous range of a grouped order that
// walks GROUP_M tile rows column by column, so the tiles one XCD runs at a time share a few
// activation and weight panels in its L2.
constexpr int GROUP_M = 8;

__device__ __forceinline__ void tile_of(int b, int G, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int q = G / 8, r = G % 8, x = b % 8, l = b / 8;
  const int p = x < r ? x * (q + 1) + l : r * (q + 1) + (x - r) * q + l;  // position in the grouped order
  const int group = p / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int rows = min(GROUP_M, tiles_m - first_m);
  const int in = p - group * GROUP_M * tiles_n;
  tm = first_m + in % rows;
  tn = in / rows;
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
struct Tile {
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = WAVES_M, WN = WAVES_N, FRAG_M = FM, FRAG_N = FN;
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;
  static constexpr int ROWS = BM + BN;  // activation rows, then weight rows, in LDS
  static constexpr int A_CPT = (BM * 4 + THREADS - 1) / THREADS;  // 16-byte code chunks per thread
  static constexpr int B_CPT = (BN * 4 + THREADS - 1) / THREADS;
  static constexpr int SA_PT = (2 * BM + THREADS - 1) / THREADS;  // (group, 4-row quad) scale words per thread
  static constexpr int SB_PT = (2 * BN + THREADS - 1) / THREADS;
  static constexpr int SCALE_BYTES = 8 * ROWS * 2;  // f16 scales laid out [group][row]
  static constexpr int STAGE_BYTES = ROWS * CODE_STRIDE + SCALE_BYTES;
  // Epilogue operands, staged in the stage buffers after the K loop: L hi and lo parts
  // [BM][EPI_RS] bf16, proj_up [BN][EPI_RS] bf16, the column scale [BN] f32 and the bias [BN] f32.
  // The rank stride holds the compiled maximum rank plus 8: 144-byte rows put the 16-byte reads
  // of 16 consecutive rows on distinct banks.
  static constexpr int EPI_RS = 64 + 8;
  static constexpr int EPI_BYTES = BM * EPI_RS * 2 * 2 + BN * EPI_RS * 2 + BN * 8;
  // Waves with 16 or more accumulator fragments (which fill the accumulation registers) finish
  // one fragment row at a time, each wave through a 32-row store region of its own placed after
  // the epilogue operands.
  static constexpr bool ROWWISE = FM * FN >= 16;
  static constexpr int EPI_LDS = EPI_BYTES + (ROWWISE ? WAVES_M * WAVES_N * 32 * FN * 64 : 0);
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES > EPI_LDS ? 2 * STAGE_BYTES : EPI_LDS;
};

// Stage a tile's epilogue operands in LDS: the column scales wcscales * wtscale and the bias
// (zero without one) when r_lo == 0, and for the ranks [r_lo, r_hi) (columns r - r_lo of the
// rank-strided arrays) the low-rank activations summed over their `parts` partial sums (in
// order) and split into bf16 hi + lo parts, and proj_up.  Padded ranks and rows past M or N are
// zero or clamped.  Each thread issues all its loads of a 16-rank block before storing any of
// them.
template <class T, bool LORA>
__device__ __forceinline__ void stage_epilogue(uint8_t* base, int rs, int r_lo, int r_hi, int t, int m0, int n0,
                                               int M, int N, int R, int parts, const float* __restrict__ lora,
                                               const uint16_t* __restrict__ pu, const uint16_t* __restrict__ wcs,
                                               const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias) {
  uint16_t* l_hi = reinterpret_cast<uint16_t*>(base);
  uint16_t* l_lo = l_hi + T::BM * rs;
  uint16_t* p_lds = l_lo + T::BM * rs;
  float* c_lds = reinterpret_cast<float*>(p_lds + T::BN * rs);
  float* b_lds = c_lds + T::BN;
  if (r_lo == 0) {
    const float ts = bf16_bits_to_f32(wts[0]);
    for (int c = t; c < T::BN; c += T::THREADS) {
      const int n = n0 + c;
      c_lds[c] = n < N ? bf16_bits_to_f32(wcs[n]) * ts : 0.0f;
      b_lds[c] = (bias != nullptr && n < N) ? bf16_bits_to_f32(bias[n]) : 0.0f;
    }
  }
  if (!LORA) return;
  constexpr int LI = (T::BM * 16 + T::THREADS - 1) / T::THREADS;
  constexpr int PI = (T::BN * 16 + T::THREADS - 1) / T::THREADS;
  if constexpr ((T::BM * 16) % T::THREADS == 0 && (T::BN * 16) % T::THREADS == 0) {
    // A tile wholly inside M x N with one partial sum and a rank that is a multiple of 16:
    // nothing is clamped, masked or summed, so every element's offset is one per-thread base plus
    // an immediate.  (Several partial sums come only with batches of at most 32 rows, whose
    // tiles are never wholly inside M.)
    if (m0 + T::BM <= M && n0 + T::BN <= N && parts == 1 && (R & 15) == 0 && r_hi <= R) {
      constexpr int RSTEP = T::THREADS / 16;  // rows per u
      const int tr = t >> 4, tc = t & 15;
      const float* lb = lora + (size_t)(m0 + tr) * R + tc;
      const uint16_t* pb = pu + (size_t)(n0 + tr) * R + tc;
      for (int r0 = r_lo; r0 < r_hi; r0 += 16) {
        float f[LI];
        uint32_t pw[PI];
#pragma unroll
        for (int u = 0; u < LI; ++u) f[u] = lb[u * RSTEP * R + r0];
#pragma unroll
        for (int u = 0; u < PI; ++u) pw[u] = pb[u * RSTEP * R + r0];
        // hi + lo split of two rows at a time with the hardware convert (nearest even)
        static_assert(LI % 2 == 0, "row pairs");
#pragma unroll
        for (int u = 0; u < LI; u += 2) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          const uint32_t hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{f[u], f[u + 1]}, bf16x2_t));
          const float e0 = f[u] - __uint_as_float(hp << 16), e1 = f[u + 1] - __uint_as_float(hp & 0xFFFF0000u);
          const uint32_t lp = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{e0, e1}, bf16x2_t));
          const int rr = tr + u * RSTEP, r = r0 - r_lo + tc;
          l_hi[rr * rs + r] = (uint16_t)hp;
          l_hi[(rr + RSTEP) * rs + r] = (uint16_t)(hp >> 16);
          l_lo[rr * rs + r] = (uint16_t)lp;  // the exact remainder, rounded
          l_lo[(rr + RSTEP) * rs + r] = (uint16_t)(lp >> 16);
        }
#pragma unroll
        for (int u = 0; u < PI; ++u) p_lds[(tr + u * RSTEP) * rs + r0 - r_lo + tc] = (uint16_t)pw[u];
      }
      return;
    }
  }
  for (int r0 = r_lo; r0 < r_hi; r0 += 16) {
    float f[LI];
    uint32_t pw[PI];
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int idx = t + u * T::THREADS;
      const int rr = min(idx >> 4, T::BM - 1), r = r0 + (idx & 15);
      const size_t at = (size_t)min(m0 + rr, M - 1) * R + (r < R ? r : 0);
      float acc_l = 0.0f;
      for (int p = 0; p < parts; ++p) acc_l += lora[(size_t)p * M * R + at];
      f[u] = r < R ? acc_l : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < PI; ++u) {
      const int idx = t + u * T::THREADS;
      const int rr = min(idx >> 4, T::BN - 1), r = r0 + (idx & 15);
      const uint32_t v = pu[(size_t)min(n0 + rr, N - 1) * R + (r < R ? r : 0)];
      pw[u] = r < R ? v : 0u;
    }
#pragma unroll
    for (int u = 0; u < LI; ++u) {
      const int idx = t + u * T::THREADS;
      if ((T::BM * 16) % T::THREADS == 0 || idx < T::BM * 16) {
        const int rr = idx >> 4, r = r0 - r_lo + (idx & 15);
        const uint32_t hb = f32_to_bf16_bits(f[u]);
        l_hi[rr * rs + r] = (uint16_t)hb;
        l_lo[rr * rs + r] = (uint16_t)f32_to_bf16_bits(f[u] - bf16_bits_to_f32(hb));  // exact remainder
      }
    }
#pragma unroll
    for (int u = 0; u < PI; ++u) {
      const int idx = t + u * T::THREADS;
      if ((T::BN * 16) % T::THREADS == 0 || idx < T::BN * 16) p_lds[(idx >> 4) * rs + r0 - r_lo + (idx & 15)] = (uint16_t)pw[u];
    }
  }
}

// Two float32 -> packed bf16 pair, round to nearest even (hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = __builtin_convertvector(float2_t{a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Wait until at most N vector-memory operations of this wave are outstanding and all its LDS
// operations are done, then join the workgroup barrier.  The compiler may not move memory
// operations across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Epilogue of a tile: stage the operands in LDS (`lds` must be free; it is left in use), then
// acc *= wcscales[n] * wtscale, add L @ proj_up^T on the matrix cores, round to bf16 and store.
// acc[i][j][4q + e] is y[m, n] with m = mb + i*32 + l32, n = nb + j*32 + 8q + 4h + e.
template <class T, bool LORA>
__device__ __forceinline__ void epilogue(float16_t (&acc)[T::FRAG_M][T::FRAG_N], uint8_t* lds, int t, int m0,
                                         int n0, int M, int N, int R, int parts, const float* __restrict__ lora,
                                         const uint16_t* __restrict__ pu, const uint16_t* __restrict__ wcs,
                                         const uint16_t* __restrict__ wts, const uint16_t* __restrict__ bias,
                                         uint16_t* __restrict__ y) {
  constexpr int FM = T::FRAG_M, FN = T::FRAG_N;
  constexpr int rs = T::EPI_RS;  // rank stride of the staged operands
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int l32 = lane & 31, h = lane >> 5;
  const int rp = LORA ? 16 * ((R + 15) / 16) : 0;  // padded rank
  stage_epilogue<T, LORA>(lds, rs, 0, rp, t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias);
  __syncthreads();
  const int mb = m0 + wm * FM * 32, nb = n0 + wn * FN * 32;
  const uint16_t* l_hi = reinterpret_cast<const uint16_t*>(lds);
  const uint16_t* l_lo = l_hi + T::BM * rs;
  const uint16_t* p_lds = l_lo + T::BM * rs;
  const float* c_lds = reinterpret_cast<const float*>(p_lds + T::BN * rs);
  const float* b_lds = c_lds + T::BN;
  const bool has_bias = bias != nullptr;
  if constexpr (T::ROWWISE) {
    // Same arithmetic, in the same order per element, one fragment at a time; each fragment
    // row then leaves through the wave's store region (16-byte stores) or, when y rows are not
    // whole 16-byte runs, directly.
    constexpr int RSB = FN * 64, CPR = FN * 4;
    uint8_t* reg = lds + T::EPI_BYTES + wave * 32 * RSB;
    const bool coalesce = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    const bool n4 = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * FM * 32 + i * 32 + l32;
      const int m = mb + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float16_t a = acc[i][j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4_t c = *reinterpret_cast<const float4_t*>(c_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[4 * q + e] *= c[e];
        }
        if (LORA) {
          for (int r0 = 0; r0 < rp; r0 += 16) {
            const bf16x8_t pv =
                *reinterpret_cast<const bf16x8_t*>(p_lds + (wn * FN * 32 + j * 32 + l32) * rs + r0 + 8 * h);
            const bf16x8_t lhi = *reinterpret_cast<const bf16x8_t*>(l_hi + row * rs + r0 + 8 * h);
            const bf16x8_t llo = *reinterpret_cast<const bf16x8_t*>(l_lo + row * rs + r0 + 8 * h);
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv, lhi, a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv, llo, a, 0, 0, 0);
          }
        }
        if (has_bias) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4_t b = *reinterpret_cast<const float4_t*>(b_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * q + e] += b[e];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p0 = pack_bf16x2(a[4 * q], a[4 * q + 1]);
          const uint32_t p1 = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
          const int n = nb + j * 32 + 8 * q + 4 * h;
          if (coalesce) {
            const int ch = 4 * j + q;
            *reinterpret_cast<u32x2_t*>(reg + l32 * RSB + 16 * ((ch + (l32 >> 1)) % CPR) + 8 * h) = u32x2_t{p0, p1};
          } else if (m < M) {
            uint16_t* yrow = y + (size_t)m * N;
            if (n4) {
              if (n < N) *reinterpret_cast<u32x2_t*>(yrow + n) = u32x2_t{p0, p1};
            } else {
              const uint16_t v[4] = {(uint16_t)p0, (uint16_t)(p0 >> 16), (uint16_t)p1, (uint16_t)(p1 >> 16)};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) yrow[n + e] = v[e];
            }
          }
        }
      }
      if (coalesce) {
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < CPR / 2; ++it) {
          const int c = it * 64 + lane, r = c / CPR, ch = c % CPR;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reg + r * RSB + 16 * ((ch + (r >> 1)) % CPR));
          const int mr = mb + i * 32 + r, n = nb + 8 * ch;
          if (mr < M && n < N) *reinterpret_cast<u32x4_t*>(y + (size_t)mr * N + n) = v;
        }
        wave_lds_sync();  // the region is rewritten by the next fragment row
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4_t c = *reinterpret_cast<const float4_t*>(c_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[i][j][4 * q + e] *= c[e];
    }
  if (LORA) {
    for (int r0 = 0; r0 < rp; r0 += 16) {
      bf16x8_t pv[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        pv[j] = *reinterpret_cast<const bf16x8_t*>(p_lds + (wn * FN * 32 + j * 32 + l32) * rs + r0 + 8 * h);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * FM * 32 + i * 32 + l32;
        const bf16x8_t lhi = *reinterpret_cast<const bf16x8_t*>(l_hi + row * rs + r0 + 8 * h);
        const bf16x8_t llo = *reinterpret_cast<const bf16x8_t*>(l_lo + row * rs + r0 + 8 * h);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv[j], lhi, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv[j], llo, acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  if (has_bias) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4_t b = *reinterpret_cast<const float4_t*>(b_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j][4 * q + e] += b[e];
      }
  }
  if ((N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
    // Coalesced stores: each wave passes its rounded tile through a private LDS region (IC fragment
    // rows at a time) and writes whole 16-byte runs of y rows (a wave instruction covers
    // 64 / CPR rows x 64 FN contiguous bytes).  Chunk ch of region row r sits at position
    // (ch + r / 2) % CPR, which keeps both the 8-byte writes and the 16-byte reads on distinct banks.
    constexpr int WAVES = T::WM * T::WN;
    constexpr int RSB = FN * 64;  // bytes per region row
    constexpr int CPR = FN * 4;   // 16-byte chunks per region row
    constexpr int IC = WAVES * FM * 32 * RSB <= T::EPI_BYTES ? FM
                       : ((FM % 2) == 0 && WAVES * (FM / 2) * 32 * RSB <= T::EPI_BYTES) ? FM / 2 : 1;
    static_assert(WAVES * IC * 32 * RSB <= T::EPI_BYTES, "store regions fit the epilogue's LDS");
    __syncthreads();  // every wave is done with the staged operands
    uint8_t* reg = lds + wave * IC * 32 * RSB;
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += IC) {
#pragma unroll
      for (int i = i0; i < i0 + IC; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = (i - i0) * 32 + l32, ch = 4 * j + q;
            const uint32_t p0 = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            const uint32_t p1 = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<u32x2_t*>(reg + r * RSB + 16 * ((ch + (r >> 1)) % CPR) + 8 * h) = u32x2_t{p0, p1};
          }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < IC * CPR / 2; ++it) {
        const int c = it * 64 + lane, r = c / CPR, ch = c % CPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(reg + r * RSB + 16 * ((ch + (r >> 1)) % CPR));
        const int m = mb + i0 * 32 + r, n = nb + 8 * ch;
        if (m < M && n < N) *reinterpret_cast<u32x4_t*>(y + (size_t)m * N + n) = v;
      }
      wave_lds_sync();  // the region is rewritten by the next fragment rows
    }
    return;
  }
  const bool n4 = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = mb + i * 32 + l32;
    if (m >= M) continue;
    uint16_t* yrow = y + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb + j * 32 + 8 * q + 4 * h;
        const uint32_t p0 = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        const uint32_t p1 = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        if (n4) {
          if (n < N) *reinterpret_cast<u32x2_t*>(yrow + n) = u32x2_t{p0, p1};
        } else {
          const uint16_t v[4] = {(uint16_t)p0, (uint16_t)(p0 >> 16), (uint16_t)p1, (uint16_t)(p1 >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yrow[n + e] = v[e];
        }
      }
  }
}

// 16-byte chunk position of a code row's chunk 0 in LDS (chunk c goes to c ^ code_swizzle(r)):
// rows r and r + 4 share banks (64-byte rows, 256 bytes of banks), so the four rows of a bank
// line take distinct positions.
__device__ __forceinline__ int code_swizzle(int row) { return (row >> 2) & 3; }

// Issue one K-step's direct loads of a wave: ROUNDS code instructions (16 bytes per lane) and
// SROUNDS scale instructions (4 bytes per lane) into the stage at `stage`.
template <class D>
__device__ __forceinline__ void dma_issue(uint8_t* stage, int wave, uint32_t kb0, size_t g0,
                                          const uint8_t* const* c_base, const uint32_t* c_off,
                                          const uint8_t* const* s_base, const uint32_t* s_off,
                                          const uint32_t* s_stride) {
#pragma unroll
  for (int r = 0; r < D::ROUNDS; ++r)
    __builtin_amdgcn_global_load_lds(c_base[r] + kb0 + c_off[r],
                                     (lds_void*)(stage + (r * D::ROUND_ROWS + wave * 16) * 64), 16, 0, 0);
#pragma unroll
  for (int r = 0; r < D::SROUNDS; ++r)
    __builtin_amdgcn_global_load_lds(s_base[r] + g0 * s_stride[r] + s_off[r],
                                     (lds_void*)(stage + D::SCALE_OFF + (r * D::WAVES + wave) * 256), 4, 0, 0);
}

// (the persistent form and its epilogue)
template <class T, class D>
struct PersistTile {
  static constexpr int RW = 32;      // ranks staged per pass
  static constexpr int RS = RW + 8;  // rank stride of the staged operands: 80-byte rows put the 16-byte
                                     // reads of 16 consecutive rows on distinct banks
  static constexpr int WAVES = T::WM * T::WN;
  static constexpr int RSB = T::FRAG_N * 64, CPR = T::FRAG_N * 4;  // store region row: bytes, 16-byte chunks
  static constexpr int OPS = T::BM * RS * 4 + T::BN * RS * 2 + T::BN * 8;  // L hi + lo, proj_up, scale, bias
  static constexpr int REGIONS = WAVES * 32 * RSB;  // one 32-row fragment row per wave
  static constexpr int E_OFF = 2 * D::STAGE;
  static constexpr int E_BYTES = OPS > REGIONS ? OPS : REGIONS;
  static constexpr int LDS_BYTES = 3 * D::STAGE > E_OFF + E_BYTES ? 3 * D::STAGE : E_OFF + E_BYTES;
  static constexpr int ST = T::FRAG_M * CPR / 2;  // y stores of a wave per tile
  static_assert(!T::ROWWISE, "whole-tile epilogue");
  static_assert(D::LOADS + ST < 64, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

// N buffer stores that the hardware drops (offsets from 2^31 up, past any y the persistent kernels
// accept), each to its own offset so that none is merged with another.
template <int N>
__device__ __forceinline__ void drop_stores(__amdgpu_buffer_rsrc_t yr) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, yr, (int)(0x80000000u + 16u * (uint32_t)i), 0, 0);
}

// LDS-only barrier: waits for this wave's LDS operations, not for its loads or stores in flight.
__device__ __forceinline__ void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Epilogue of one tile in the persistent kernels (as `epilogue`, whole-tile form): the operands are
// staged in a region E after stage slots 0 and 1, 32 ranks per pass; `prefetch` runs first (it
// issues the next tile's first K-steps into slots 0 and 1); y leaves through
// exactly P::ST buffer stores per wave, chunks outside y at an offset the hardware drops.
template <class T, class P, bool LORA, class Prefetch>
__device__ __forceinline__ void persist_epilogue(float16_t (&acc)[T::FRAG_M][T::FRAG_N], uint8_t* lds, int wave, int lane,
                                                 int m0, int n0, int M, int N, int R, int parts,
                                                 const float* __restrict__ lora, const uint16_t* __restrict__ pu,
                                                 const uint16_t* __restrict__ wcs, const uint16_t* __restrict__ wts,
                                                 const uint16_t* __restrict__ bias, __amdgpu_buffer_rsrc_t yr,
                                                 Prefetch&& prefetch) {
  constexpr int FM = T::FRAG_M, FN = T::FRAG_N;
  constexpr int rw = P::RW, rs = P::RS, RSB = P::RSB, CPR = P::CPR;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int l32 = lane & 31, h = lane >> 5;
  const int t = wave * 64 + lane;
  const int rp = LORA ? 16 * ((R + 15) / 16) : 0;  // padded rank
  uint8_t* const E = lds + P::E_OFF;
  const uint16_t* l_hi = reinterpret_cast<const uint16_t*>(E);
  const uint16_t* l_lo = l_hi + T::BM * rs;
  const uint16_t* p_lds = l_lo + T::BM * rs;
  const float* c_lds = reinterpret_cast<const float*>(p_lds + T::BN * rs);
  const float* b_lds = c_lds + T::BN;
  // the caller's prefetch of the next tile's first K-steps into slots 0 and 1 (free since the K
  // loop's last barrier), then the epilogue operands' first pass into E, whose loads wait out
  // the same latency
  prefetch();
  stage_epilogue<T, LORA>(E, rs, 0, min(rp, rw), t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias);
  lds_only_barrier();

  // acc *= wcscales * wtscale; + L @ proj_up^T (passes of 32 ranks); + bias (as in `epilogue`)
  const int mb = m0 + wm * FM * 32, nb = n0 + wn * FN * 32;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4_t c = *reinterpret_cast<const float4_t*>(c_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[i][j][4 * q + e] *= c[e];
    }
  if (LORA) {
    for (int lo = 0; lo < rp; lo += rw) {
      if (lo > 0) {
        lds_only_barrier();  // every wave is done with the previous pass
        stage_epilogue<T, LORA>(E, rs, lo, min(rp, lo + rw), t, m0, n0, M, N, R, parts, lora, pu, wcs, wts, bias);
        lds_only_barrier();
      }
      for (int r0 = 0; r0 < min(rp - lo, rw); r0 += 16) {
        bf16x8_t pv[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
          pv[j] = *reinterpret_cast<const bf16x8_t*>(p_lds + (wn * FN * 32 + j * 32 + l32) * rs + r0 + 8 * h);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * FM * 32 + i * 32 + l32;
          const bf16x8_t lhi = *reinterpret_cast<const bf16x8_t*>(l_hi + row * rs + r0 + 8 * h);
          const bf16x8_t llo = *reinterpret_cast<const bf16x8_t*>(l_lo + row * rs + r0 + 8 * h);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv[j], lhi, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pv[j], llo, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
  if (bias != nullptr) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4_t b = *reinterpret_cast<const float4_t*>(b_lds + wn * FN * 32 + j * 32 + 8 * q + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < FM; ++i) acc[i][j][4 * q + e] += b[e];
      }
  }
  lds_only_barrier();  // every wave is done with the staged operands: E becomes store regions

  // one fragment row at a time through the wave's region (chunk ch of region row r at
  // (ch + r / 2) % CPR), then whole 16-byte runs of y rows
  uint8_t* reg = E + wave * 32 * RSB;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = 4 * j + q;
        const uint32_t p0 = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        const uint32_t p1 = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        *reinterpret_cast<u32x2_t*>(reg + l32 * RSB + 16 * ((ch + (l32 >> 1)) % CPR) + 8 * h) = u32x2_t{p0, p1};
      }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < CPR / 2; ++it) {
      const int c = it * 64 + lane, r = c / CPR, ch = c % CPR;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(reg + r * RSB + 16 * ((ch + (r >> 1)) % CPR));
      const int m = mb + i * 32 + r, n = nb + 8 * ch;
      const uint32_t off = (m < M && n < N) ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 2u : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(val, yr, (int)off, 0, 0);
    }
    wave_lds_sync();  // the region is rewritten by the next fragment row
  }
}

}  // namespace

}  // namespace w4a4
