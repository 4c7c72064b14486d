// W_KV = W_K^-1 . W_V on the host in float64 (Slim Attention article,
// localbendi.com, section "K-Cache is All You Need": the new parameter
// matrix, computed once per layer).
//
// Right-looking blocked LU factorisation of W_K with partial pivoting (rows
// swapped in W_K and in the right-hand sides W_V together), then blocked
// forward and back substitution for all d right-hand sides.  The O(d^3)
// work is in rank-k updates C -= A.B that run on std::threads over row
// blocks of C with a cache-blocked i-k-j loop.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>
#include <stdint.h>

namespace slim {

int host_threads() {
  const char* e = std::getenv("SLIM_HOST_THREADS");
  int n = e ? std::atoi(e) : 0;
  if (n <= 0) {
    n = (int)std::thread::hardware_concurrency();
    if (n <= 0) n = 1;
    n = std::min(n, 16);
  }
  return n;
}

template <class F>
static void parallel_rows(int lo, int hi, int grain, F f) {
  const int n = hi - lo;
  if (n <= 0) return;
  int nt = std::min(host_threads(), (n + grain - 1) / grain);
  if (nt <= 1) {
    f(lo, hi);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(nt);
  for (int t = 0; t < nt; ++t) {
    const int a = lo + (int)((long long)n * t / nt), b = lo + (int)((long long)n * (t + 1) / nt);
    th.emplace_back([=] { f(a, b); });
  }
  for (auto& x : th) x.join();
}

// C[m x n] -= A[m x k] . B[k x n]   (row-major, leading dimensions given)
static void gemm_sub(int m, int n, int k, const double* A, int lda, const double* B, int ldb,
                     double* C, int ldc) {
  if (m <= 0 || n <= 0 || k <= 0) return;
  parallel_rows(0, m, 8, [&](int i0, int i1) {
    constexpr int KB = 128, NB = 512;
    for (int kk = 0; kk < k; kk += KB) {
      const int ke = std::min(k, kk + KB);
      for (int jj = 0; jj < n; jj += NB) {
        const int je = std::min(n, jj + NB);
        for (int i = i0; i < i1; ++i) {
          double* __restrict__ c = C + (size_t)i * ldc;
          const double* a = A + (size_t)i * lda;
          for (int p = kk; p < ke; ++p) {
            const double av = a[p];
            if (av == 0.0) continue;
            const double* __restrict__ b = B + (size_t)p * ldb;
            for (int j = jj; j < je; ++j) c[j] -= av * b[j];
          }
        }
      }
    }
  });
}

// Solves A X = R in place: A [d x d] is overwritten by its LU factors, R
// [d x nr] by X.  Returns false on a zero pivot.
bool lu_solve_inplace(double* A, double* R, int d, int nr) {
  const int nb = 64;
  std::vector<double> tmp(std::max(d, nr));
  for (int k0 = 0; k0 < d; k0 += nb) {
    const int k1 = std::min(d, k0 + nb);
    // panel: columns k0..k1-1, rows k0..d-1
    for (int k = k0; k < k1; ++k) {
      int piv = k;
      double best = std::fabs(A[(size_t)k * d + k]);
      for (int i = k + 1; i < d; ++i) {
        const double v = std::fabs(A[(size_t)i * d + k]);
        if (v > best) {
          best = v;
          piv = i;
        }
      }
      if (!(best > 0.0)) return false;
      if (piv != k) {
        std::memcpy(tmp.data(), A + (size_t)k * d, sizeof(double) * d);
        std::memcpy(A + (size_t)k * d, A + (size_t)piv * d, sizeof(double) * d);
        std::memcpy(A + (size_t)piv * d, tmp.data(), sizeof(double) * d);
        std::memcpy(tmp.data(), R + (size_t)k * nr, sizeof(double) * nr);
        std::memcpy(R + (size_t)k * nr, R + (size_t)piv * nr, sizeof(double) * nr);
        std::memcpy(R + (size_t)piv * nr, tmp.data(), sizeof(double) * nr);
      }
      const double inv = 1.0 / A[(size_t)k * d + k];
      const double* rk = A + (size_t)k * d;
      parallel_rows(k + 1, d, 256, [&](int i0, int i1) {
        for (int i = i0; i < i1; ++i) {
          double* ri = A + (size_t)i * d;
          const double l = ri[k] * inv;
          ri[k] = l;
          for (int j = k + 1; j < k1; ++j) ri[j] -= l * rk[j];
        }
      });
    }
    if (k1 < d) {
      // U12 = L11^-1 A12 (unit lower triangular), parallel over columns
      const int nc = d - k1;
      const int nt = std::min(host_threads(), (nc + 63) / 64);
      std::vector<std::thread> th;
      for (int t = 0; t < nt; ++t) {
        const int c0 = k1 + (int)((long long)nc * t / nt), c1 = k1 + (int)((long long)nc * (t + 1) / nt);
        th.emplace_back([=] {
          for (int k = k0; k < k1; ++k) {
            const double* rk = A + (size_t)k * d;
            for (int i = k + 1; i < k1; ++i) {
              double* ri = A + (size_t)i * d;
              const double l = ri[k];
              for (int j = c0; j < c1; ++j) ri[j] -= l * rk[j];
            }
          }
        });
      }
      for (auto& x : th) x.join();
      // A22 -= L21 . U12
      gemm_sub(d - k1, d - k1, k1 - k0, A + (size_t)k1 * d + k0, d, A + (size_t)k0 * d + k1, d,
               A + (size_t)k1 * d + k1, d);
    }
  }
  // forward substitution L Y = R (unit lower), blocked by rows
  for (int i0 = 0; i0 < d; i0 += nb) {
    const int i1 = std::min(d, i0 + nb);
    gemm_sub(i1 - i0, nr, i0, A + (size_t)i0 * d, d, R, nr, R + (size_t)i0 * nr, nr);
    for (int i = i0; i < i1; ++i) {
      double* ri = R + (size_t)i * nr;
      for (int k = i0; k < i; ++k) {
        const double l = A[(size_t)i * d + k];
        const double* rk = R + (size_t)k * nr;
        for (int j = 0; j < nr; ++j) ri[j] -= l * rk[j];
      }
    }
  }
  // back substitution U X = Y, blocked by rows from the bottom
  for (int i1 = d; i1 > 0; i1 -= nb) {
    const int i0 = std::max(0, i1 - nb);
    gemm_sub(i1 - i0, nr, d - i1, A + (size_t)i0 * d + i1, d, R + (size_t)i1 * nr, nr,
             R + (size_t)i0 * nr, nr);
    for (int i = i1 - 1; i >= i0; --i) {
      double* ri = R + (size_t)i * nr;
      for (int k = i + 1; k < i1; ++k) {
        const double u = A[(size_t)i * d + k];
        const double* rk = R + (size_t)k * nr;
        for (int j = 0; j < nr; ++j) ri[j] -= u * rk[j];
      }
      const double inv = 1.0 / A[(size_t)i * d + i];
      for (int j = 0; j < nr; ++j) ri[j] *= inv;
    }
  }
  return true;
}

// float64 -> bfloat16 bits, round to nearest even (correct rounding: the
// intermediate float32 is rounded to odd so no double rounding occurs).
uint16_t f64_to_bf16_rne(double x) {
  if (std::isnan(x)) return 0x7fc0;
  float f = (float)x;
  if (std::isinf(f) && !std::isinf(x)) {
    // overflowed float32: the bf16 result is the infinity of that sign
  } else if (std::fabs((double)f) > std::fabs(x)) {
    f = std::nextafter(f, 0.0f);
  }
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((double)f != x && !std::isinf(f)) u |= 1u;  // sticky bit (round to odd)
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

}  // namespace slim
