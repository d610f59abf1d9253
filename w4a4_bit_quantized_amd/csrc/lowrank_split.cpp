// Offline low-rank split of a smoothed weight ("SVDQuant W4A4" page, "Overview": four-bit
// weights and activations with a small low-rank branch that corrects part of the quantization
// error; "Checkpoint contract": proj_down (K, R), proj_up (N, R)).  Host code, run once per
// checkpoint; the online layer never calls it.
//
//   W_s       = W * smooth_factor                 (float64, exact for bf16 inputs)
//   W_s      ~= U S V^T restricted to the top R singular triplets
//   proj_up   = bf16(U_R sqrt(S_R)),  proj_down = bf16(V_R sqrt(S_R))
//   residual  = bf16(W_s - proj_up proj_down^T)   (against the stored bf16 factors)
//
// The top-R triplets come from a randomized range finder (Halko, Martinsson and Tropp,
// "Finding structure with randomness", 2011, algorithms 4.4 and 5.1): Y = W_s Omega with a
// Gaussian test matrix of R + p columns, q power iterations with re-orthonormalization between
// the products, B = Q^T W_s, and an SVD of the small factor B by one-sided Jacobi rotations
// (Hestenes) on B^T.  Orthonormalization is modified Gram-Schmidt, applied twice.  Omega is
// drawn from SplitMix64 (Steele, Lea and Flood, 2014) on the counter seed * 2^32 + index, with
// the Box-Muller transform.  The large products run on `threads` host threads over row blocks.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "w4a4.h"

namespace {

double bf16_to_double(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Round to nearest even, from double directly (one rounding); overflow to infinity.
uint16_t double_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const double a = std::fabs(v);
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                       // a = f * 2^e, f in [0.5, 1)
  int ex = std::max(e - 1, -126);          // subnormals share the 2^-126 grid
  const double ulp = std::ldexp(1.0, ex - 7);
  double q = a / ulp;                      // exact: power-of-two scaling
  double r = std::nearbyint(q);            // ties to even (default rounding mode)
  double rv = r * ulp;
  float f = (float)rv;                     // exact: rv has at most 8 significant bits
  if (!(std::fabs(f) <= 3.3895313892515355e38)) return sign | 0x7F80;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

double gaussian(uint64_t seed, uint64_t i) {
  // two uniforms in (0, 1] from 53-bit draws, Box-Muller
  const double u1 = ((double)(splitmix64((seed << 32) ^ (2 * i)) >> 11) + 1.0) * 0x1.0p-53;
  const double u2 = (double)(splitmix64((seed << 32) ^ (2 * i + 1)) >> 11) * 0x1.0p-53;
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}

template <class F>
void parallel_rows(int64_t n, int threads, F f) {
  const int t = (int)std::max<int64_t>(1, std::min<int64_t>(threads, n));
  if (t == 1) {
    f(0, n);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t chunk = (n + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    const int64_t a = i * chunk, b = std::min(n, a + chunk);
    if (a < b) pool.emplace_back([=] { f(a, b); });
  }
  for (auto& th : pool) th.join();
}

// C (rows x l) = A (rows x K, row-major) * X (K x l, row-major)
void mul_ax(const std::vector<double>& A, int64_t rows, int64_t K, const std::vector<double>& X, int64_t l,
            std::vector<double>& C, int threads) {
  C.assign((size_t)rows * l, 0.0);
  parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
    for (int64_t n = a; n < b; ++n) {
      double* c = &C[(size_t)n * l];
      const double* arow = &A[(size_t)n * K];
      for (int64_t k = 0; k < K; ++k) {
        const double v = arow[k];
        const double* x = &X[(size_t)k * l];
        for (int64_t j = 0; j < l; ++j) c[j] += v * x[j];
      }
    }
  });
}

// C (K x l) = A^T (K x rows) * Y (rows x l): each thread owns a block of K columns of A
void mul_aty(const std::vector<double>& A, int64_t rows, int64_t K, const std::vector<double>& Y, int64_t l,
             std::vector<double>& C, int threads) {
  C.assign((size_t)K * l, 0.0);
  parallel_rows(K, threads, [&](int64_t a, int64_t b) {
    for (int64_t n = 0; n < rows; ++n) {
      const double* arow = &A[(size_t)n * K];
      const double* y = &Y[(size_t)n * l];
      for (int64_t k = a; k < b; ++k) {
        const double v = arow[k];
        double* c = &C[(size_t)k * l];
        for (int64_t j = 0; j < l; ++j) c[j] += v * y[j];
      }
    }
  });
}

// Orthonormalize the l columns of Y (rows x l, row-major) in place: modified Gram-Schmidt, twice.
// A column that vanishes is replaced by zeros (it then carries no direction).
void orthonormalize(std::vector<double>& Y, int64_t rows, int64_t l) {
  for (int pass = 0; pass < 2; ++pass) {
    for (int64_t j = 0; j < l; ++j) {
      for (int64_t i = 0; i < j; ++i) {
        double d = 0.0;
        for (int64_t n = 0; n < rows; ++n) d += Y[(size_t)n * l + i] * Y[(size_t)n * l + j];
        for (int64_t n = 0; n < rows; ++n) Y[(size_t)n * l + j] -= d * Y[(size_t)n * l + i];
      }
      double nn = 0.0;
      for (int64_t n = 0; n < rows; ++n) nn += Y[(size_t)n * l + j] * Y[(size_t)n * l + j];
      const double inv = nn > 0.0 ? 1.0 / std::sqrt(nn) : 0.0;
      for (int64_t n = 0; n < rows; ++n) Y[(size_t)n * l + j] *= inv;
    }
  }
}

}  // namespace

extern "C" w4a4_status svdq_lowrank_split(const void* w, const void* smooth_factor, int64_t N, int64_t K, int64_t R,
                                          int32_t oversample, int32_t power_iters, uint64_t seed, int32_t threads,
                                          void* proj_down, void* proj_up, void* residual, float* singular_values) {
  if (N < 1 || K < 1 || R < 0 || R > W4A4_MAX_RANK || R > std::min(N, K) || oversample < 0 || power_iters < 0 ||
      N > ((int64_t)1 << 20) || K > ((int64_t)1 << 20) || N * K > ((int64_t)1 << 31))
    return W4A4_ERR_SHAPE;
  if (!w || !smooth_factor || !residual || (R > 0 && (!proj_down || !proj_up))) return W4A4_ERR_NULL;
  if (threads <= 0) threads = (int32_t)std::max(1u, std::thread::hardware_concurrency());
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  const uint16_t* lb = static_cast<const uint16_t*>(smooth_factor);
  uint16_t* pd = static_cast<uint16_t*>(proj_down);
  uint16_t* pu = static_cast<uint16_t*>(proj_up);
  uint16_t* rs = static_cast<uint16_t*>(residual);

  std::vector<double> ws((size_t)N * K);
  parallel_rows(N, threads, [&](int64_t a, int64_t b) {
    for (int64_t n = a; n < b; ++n)
      for (int64_t k = 0; k < K; ++k)
        ws[(size_t)n * K + k] = bf16_to_double(wb[(size_t)n * K + k]) * bf16_to_double(lb[k]);
  });
  if (R == 0) {
    for (size_t i = 0; i < ws.size(); ++i) rs[i] = double_to_bf16(ws[i]);
    return W4A4_OK;
  }
  const int64_t l = std::min<int64_t>(R + oversample, std::min(N, K));

  // range finder with power iterations
  std::vector<double> omega((size_t)K * l), Y, Z;
  for (size_t i = 0; i < omega.size(); ++i) omega[i] = gaussian(seed, i);
  mul_ax(ws, N, K, omega, l, Y, threads);
  orthonormalize(Y, N, l);
  for (int it = 0; it < power_iters; ++it) {
    mul_aty(ws, N, K, Y, l, Z, threads);  // Z = W_s^T Y
    orthonormalize(Z, K, l);
    mul_ax(ws, N, K, Z, l, Y, threads);   // Y = W_s Z
    orthonormalize(Y, N, l);
  }
  // A = B^T = W_s^T Q (K x l); one-sided Jacobi: A V = U S with orthogonal columns
  std::vector<double> A;
  mul_aty(ws, N, K, Y, l, A, threads);
  std::vector<double> V((size_t)l * l, 0.0);
  for (int64_t i = 0; i < l; ++i) V[(size_t)i * l + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double off = 0.0;
    for (int64_t i = 0; i < l - 1; ++i)
      for (int64_t j = i + 1; j < l; ++j) {
        double alpha = 0.0, beta = 0.0, gamma = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double ai = A[(size_t)k * l + i], aj = A[(size_t)k * l + j];
          alpha += ai * ai;
          beta += aj * aj;
          gamma += ai * aj;
        }
        if (gamma == 0.0 || std::fabs(gamma) <= 1e-15 * std::sqrt(alpha * beta)) continue;
        off = std::max(off, std::fabs(gamma) / std::sqrt(alpha * beta));
        const double zeta = (beta - alpha) / (2.0 * gamma);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int64_t k = 0; k < K; ++k) {
          const double ai = A[(size_t)k * l + i], aj = A[(size_t)k * l + j];
          A[(size_t)k * l + i] = c * ai - s * aj;
          A[(size_t)k * l + j] = s * ai + c * aj;
        }
        for (int64_t k = 0; k < l; ++k) {
          const double vi = V[(size_t)k * l + i], vj = V[(size_t)k * l + j];
          V[(size_t)k * l + i] = c * vi - s * vj;
          V[(size_t)k * l + j] = s * vi + c * vj;
        }
      }
    if (off <= 1e-14) break;
  }
  // singular values = column norms of A; order descending
  std::vector<double> sig(l);
  for (int64_t j = 0; j < l; ++j) {
    double nn = 0.0;
    for (int64_t k = 0; k < K; ++k) nn += A[(size_t)k * l + j] * A[(size_t)k * l + j];
    sig[j] = std::sqrt(nn);
  }
  std::vector<int64_t> order(l);
  for (int64_t j = 0; j < l; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return sig[a] > sig[b]; });

  // W_s ~= Q B = (Q V) S (A S^-1)^T: left vectors Q V, right vectors A / S
  std::vector<double> pu_d((size_t)N * R), pd_d((size_t)K * R);
  for (int64_t r = 0; r < R; ++r) {
    const int64_t j = order[r];
    const double sv = sig[j], root = std::sqrt(sv), inv = sv > 0 ? 1.0 / sv : 0.0;
    if (singular_values) singular_values[r] = (float)sv;
    for (int64_t k = 0; k < K; ++k) {
      const uint16_t b = double_to_bf16(A[(size_t)k * l + j] * inv * root);
      pd[(size_t)k * R + r] = b;
      pd_d[(size_t)k * R + r] = bf16_to_double(b);
    }
    parallel_rows(N, threads, [&](int64_t a, int64_t b) {
      for (int64_t n = a; n < b; ++n) {
        double u = 0.0;
        for (int64_t i = 0; i < l; ++i) u += Y[(size_t)n * l + i] * V[(size_t)i * l + j];
        const uint16_t bb = double_to_bf16(u * root);
        pu[(size_t)n * R + r] = bb;
        pu_d[(size_t)n * R + r] = bf16_to_double(bb);
      }
    });
  }
  // residual against the stored bf16 factors
  parallel_rows(N, threads, [&](int64_t a, int64_t b) {
    for (int64_t n = a; n < b; ++n)
      for (int64_t k = 0; k < K; ++k) {
        double v = ws[(size_t)n * K + k];
        for (int64_t r = 0; r < R; ++r) v -= pu_d[(size_t)n * R + r] * pd_d[(size_t)k * R + r];
        rs[(size_t)n * K + k] = double_to_bf16(v);
      }
  });
  return W4A4_OK;
}
