// Comparison of GPU results with the oracle's fp64 values.
//
// TEST INFRASTRUCTURE ONLY, built into the oracle's library. It computes
// error statistics; it holds none of the gate's arithmetic.
//
// Conventions: a bf16 result is compared with the oracle's fp64 value
// rounded once to bf16 (nearest, ties to even). The distance in ulps between
// two bf16 values is the difference of their positions on the ordered line
// of bf16 values (+0 and -0 share a position).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

extern "C" void oracle_round_bf16(const double* v, int64_t n, uint16_t* out);

namespace {

double widen(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

int64_t ordered(uint16_t bits) {
  int64_t mag = bits & 0x7FFF;
  return (bits & 0x8000) ? -mag : mag;
}

template <class F>
void split_rows(int64_t rows, int nthreads, F fn) {
  nthreads = std::max(1, (int)std::min<int64_t>(nthreads, std::max<int64_t>(rows, 1)));
  std::vector<std::thread> pool;
  int64_t chunk = (rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = std::min(rows, (int64_t)t * chunk);
    int64_t hi = std::min(rows, lo + chunk);
    pool.emplace_back([=] { fn(t, lo, hi); });
  }
  for (auto& th : pool) th.join();
}

constexpr int kClasses = 4;
constexpr int kStats = 6;

}  // namespace

extern "C" {

// acc[c * 6 + s] for row class c (0..3) accumulates:
//   s = 0: sum (gpu - bf16(ref))^2        s = 1: sum bf16(ref)^2
//   s = 2: max ulp distance               s = 3: count of elements > 1 ulp
//   s = 4: max over rows of the row's relative L2 error
//   s = 5: count of non-finite gpu values
// row_class may be null (every row in class 0). acc is added into, so a
// caller can stream chunks of rows through it.
void oracle_compare_bf16(const uint16_t* gpu, const double* ref, int64_t rows,
                         int64_t H, const uint8_t* row_class, double* acc,
                         int nthreads) {
  nthreads = std::max(1, nthreads);
  std::vector<std::vector<double>> part(nthreads, std::vector<double>(kClasses * kStats, 0.0));
  split_rows(rows, nthreads, [&](int tid, int64_t lo, int64_t hi) {
    std::vector<uint16_t> rb(H);
    double* a = part[tid].data();
    for (int64_t t = lo; t < hi; ++t) {
      const int c = row_class ? std::min<int>(row_class[t], kClasses - 1) : 0;
      oracle_round_bf16(ref + t * H, H, rb.data());
      double e2 = 0.0, r2 = 0.0;
      for (int64_t i = 0; i < H; ++i) {
        const uint16_t gb = gpu[t * H + i];
        const double g = widen(gb), r = widen(rb[i]);
        if (!std::isfinite(g)) a[c * kStats + 5] += 1.0;
        e2 += (g - r) * (g - r);
        r2 += r * r;
        const double u = (double)std::llabs(ordered(gb) - ordered(rb[i]));
        a[c * kStats + 2] = std::max(a[c * kStats + 2], u);
        if (u > 1.0) a[c * kStats + 3] += 1.0;
      }
      a[c * kStats + 0] += e2;
      a[c * kStats + 1] += r2;
      const double rel = r2 > 0 ? std::sqrt(e2 / r2) : (e2 > 0 ? INFINITY : 0.0);
      a[c * kStats + 4] = std::max(a[c * kStats + 4], rel);
    }
  });
  for (int t = 0; t < nthreads; ++t)
    for (int j = 0; j < kClasses * kStats; ++j) {
      if (j % kStats == 2 || j % kStats == 4)
        acc[j] = std::max(acc[j], part[t][j]);
      else
        acc[j] += part[t][j];
    }
}

// The forward output check: an element passes if it is within 1 ulp of
// bf16(ref), or if |gpu - ref| <= 1e-5 |v| + 2^-24 (|x| + |gate v|) (the
// error a gate off by 1e-5 and fp32 rounding of x + gate v allow where x and
// gate * v cancel). res (added into): 0 max ulp, 1 count > 1 ulp,
// 2 count passing by the second rule, 3 count failing both.
void oracle_check_out(const uint16_t* gpu, const double* ref, const uint16_t* x,
                      const uint16_t* v, const double* gate, int64_t rows,
                      int64_t H, double* res, int nthreads) {
  nthreads = std::max(1, nthreads);
  std::vector<std::vector<double>> part(nthreads, std::vector<double>(4, 0.0));
  split_rows(rows, nthreads, [&](int tid, int64_t lo, int64_t hi) {
    std::vector<uint16_t> rb(H);
    double* a = part[tid].data();
    for (int64_t t = lo; t < hi; ++t) {
      oracle_round_bf16(ref + t * H, H, rb.data());
      for (int64_t i = 0; i < H; ++i) {
        const int64_t j = t * H + i;
        const double u = (double)std::llabs(ordered(gpu[j]) - ordered(rb[i]));
        a[0] = std::max(a[0], u);
        if (u <= 1.0) continue;
        a[1] += 1.0;
        const double xv = widen(x[j]), vv = widen(v[j]);
        const double bound = 1e-5 * std::fabs(vv) +
                             0x1p-24 * (std::fabs(xv) + std::fabs(gate[t] * vv));
        if (std::fabs(widen(gpu[j]) - ref[j]) <= bound)
          a[2] += 1.0;
        else
          a[3] += 1.0;
      }
    }
  });
  for (int t = 0; t < nthreads; ++t) {
    res[0] = std::max(res[0], part[t][0]);
    for (int j = 1; j < 4; ++j) res[j] += part[t][j];
  }
}

}  // extern "C"
