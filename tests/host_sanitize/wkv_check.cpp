// Host-side check of the W_KV solver and the float64 -> bf16 rounding,
// built with AddressSanitizer + UndefinedBehaviorSanitizer, or with
// ThreadSanitizer (the rank-k updates and the panel updates run on
// std::threads), by tests/test_host_sanitizers.py.
//
// For each size: A = diagonally dominant random matrix, X0 random, R = A.X0;
// the solver must return X with max|X - X0| small.  The bf16 rounding must
// return, for every value, the nearer of its two bf16 neighbours (the even
// one on a tie).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

namespace slim {
bool lu_solve_inplace(double* A, double* R, int d, int nr);
uint16_t f64_to_bf16_rne(double x);
}  // namespace slim

static double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

int main() {
  std::mt19937_64 rng(7);
  std::normal_distribution<double> nd(0.0, 1.0);
  const int sizes[][2] = {{1, 1}, {2, 3}, {63, 63}, {64, 64}, {65, 7}, {130, 130}, {257, 33}, {300, 300}};
  for (const auto& s : sizes) {
    const int d = s[0], nr = s[1];
    std::vector<double> A((size_t)d * d), X0((size_t)d * nr), R((size_t)d * nr, 0.0);
    for (auto& v : A) v = nd(rng);
    for (int i = 0; i < d; ++i) A[(size_t)i * d + i] += (i % 2 ? -1.0 : 1.0) * 2.0 * d;  // pivots stay well away from zero
    for (auto& v : X0) v = nd(rng);
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < d; ++k)
        for (int j = 0; j < nr; ++j) R[(size_t)i * nr + j] += A[(size_t)i * d + k] * X0[(size_t)k * nr + j];
    // rows in reverse order, so that partial pivoting has to swap
    std::vector<double> Ar((size_t)d * d), Rr((size_t)d * nr);
    for (int i = 0; i < d; ++i) {
      std::memcpy(&Ar[(size_t)i * d], &A[(size_t)(d - 1 - i) * d], sizeof(double) * d);
      std::memcpy(&Rr[(size_t)i * nr], &R[(size_t)(d - 1 - i) * nr], sizeof(double) * nr);
    }
    if (!slim::lu_solve_inplace(Ar.data(), Rr.data(), d, nr)) {
      std::printf("FAIL d=%d: reported singular\n", d);
      return 1;
    }
    double err = 0.0;
    for (size_t i = 0; i < X0.size(); ++i) err = std::fmax(err, std::fabs(Rr[i] - X0[i]));
    std::printf("d=%d nr=%d max|X-X0|=%.3e\n", d, nr, err);
    if (!(err < 1e-9)) return 1;
  }
  // a singular matrix is reported
  {
    std::vector<double> A(9, 1.0), R(3, 1.0);
    if (slim::lu_solve_inplace(A.data(), R.data(), 3, 1)) {
      std::printf("FAIL: singular matrix not reported\n");
      return 1;
    }
  }
  // bf16 rounding
  std::uniform_real_distribution<double> ud(-1.0, 1.0);
  for (int i = 0; i < 200000; ++i) {
    const double x = ud(rng) * std::ldexp(1.0, (int)(rng() % 200) - 100);
    const uint16_t b = slim::f64_to_bf16_rne(x);
    const double v = bf16_value(b);
    // neighbours of v in bf16
    const double up = bf16_value((uint16_t)(b + 1)), dn = bf16_value((uint16_t)(b - 1));
    const double e = std::fabs(v - x);
    if (e > std::fabs(up - x) || e > std::fabs(dn - x) ||
        ((e == std::fabs(up - x) || e == std::fabs(dn - x)) && (b & 1u))) {
      std::printf("FAIL bf16 rounding of %.17g -> 0x%04x\n", x, b);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}
