// Seeded synthetic inputs for the Engram gate workloads.
//
// This module draws random numbers and rounds them to bf16 / fp32. It holds
// none of the gate's arithmetic; both the fp64 oracle and the GPU library are
// fed the identical bytes it produces.
//
// Generator: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), a counter-based bijection. Counter
// words are (index_lo, index_hi, stream, draw); the key is the 64-bit seed.
// Uniforms take 53 bits of two output words and sit strictly inside (0, 1);
// normals come from the Box-Muller transform in fp64.
//
// Rounding: every value is formed in fp64 and rounded once, to bf16 by
// round-to-nearest-even or to fp32 by the C cast (also nearest-even).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t kMul0 = 0xD2511F53u;
constexpr uint32_t kMul1 = 0xCD9E8D57u;
constexpr uint32_t kWeyl0 = 0x9E3779B9u;
constexpr uint32_t kWeyl1 = 0xBB67AE85u;

inline void philox(uint32_t c[4], uint64_t seed) {
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = (uint64_t)kMul0 * c[0];
    uint64_t p1 = (uint64_t)kMul1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += kWeyl0;
    k1 += kWeyl1;
  }
}

inline void block(uint64_t seed, uint32_t stream, uint32_t draw, uint64_t idx,
                  uint32_t out[4]) {
  out[0] = (uint32_t)idx;
  out[1] = (uint32_t)(idx >> 32);
  out[2] = stream;
  out[3] = draw;
  philox(out, seed);
}

// 53 random bits -> (m + 0.5) * 2^-53, strictly inside (0, 1).
inline double unit(uint32_t hi, uint32_t lo) {
  uint64_t m = ((((uint64_t)hi) << 32) | lo) >> 11;
  return ((double)m + 0.5) * 0x1p-53;
}

inline void box_muller(const uint32_t o[4], double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unit(o[0], o[1]);
  double u2 = unit(o[2], o[3]);
  double r = std::sqrt(-2.0 * std::log(u1));
  *z0 = r * std::cos(two_pi * u2);
  *z1 = r * std::sin(two_pi * u2);
}

// Standard normal number `e` of a stream: block e/2, Box-Muller output e%2.
inline double normal_at(uint64_t seed, uint32_t stream, uint64_t e) {
  uint32_t o[4];
  block(seed, stream, 0, e >> 1, o);
  double z0, z1;
  box_muller(o, &z0, &z1);
  return (e & 1) ? z1 : z0;
}

// Student-t with 3 degrees of freedom: Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3),
// the four normals taken from two blocks of element e.
inline double student_t3_at(uint64_t seed, uint32_t stream, uint64_t e) {
  uint32_t a[4], b[4];
  block(seed, stream, 1, e, a);
  block(seed, stream, 2, e, b);
  double z, z1, z2, z3;
  box_muller(a, &z, &z1);
  box_muller(b, &z2, &z3);
  double chi2 = z1 * z1 + z2 * z2 + z3 * z3;
  return z / std::sqrt(chi2 / 3.0);
}

// fp64 -> bf16 bits, rounding once to nearest, ties to even.
inline uint16_t to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
  // bf16 keeps 8 significant bits; below 2^-126 the quantum stays 2^-133.
  int q = std::max(e - 8, -133);
  double r = std::nearbyint(std::ldexp(a, -q));  // default mode: ties to even
  double rounded = std::ldexp(r, q);
  if (rounded >= 0x1p128) return sign | 0x7F80;  // overflow to infinity
  float f = (float)rounded;                       // exact: 8 bits, in range
  uint32_t bits;
  std::memcpy(&bits, &f, 4);
  return sign | (uint16_t)((bits >> 16) & 0x7FFF);
}

template <class F>
void parallel_for(int64_t n, int nthreads, F fn) {
  if (nthreads < 1) nthreads = 1;
  if (n < 65536 || nthreads == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> pool;
  int64_t chunk = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t a = (int64_t)t * chunk, b = std::min(n, a + chunk);
    if (a >= b) break;
    pool.emplace_back([=] { fn(a, b); });
  }
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Raw Philox-4x32-10 block, for known-answer tests of the generator itself.
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                         uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox(c, ((uint64_t)key[1] << 32) | key[0]);
  std::memcpy(out, c, sizeof(c));
}

// fp64 values -> bf16 bits (exposed so the rounding can be tested).
void synth_round_bf16(const double* v, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = to_bf16(v[i]);
}

// out[i] = bf16(scale * N_i), i = 0..n-1, normals e0+i of `stream`.
void synth_normal_bf16(uint64_t seed, uint32_t stream, int64_t e0, int64_t n,
                       double scale, uint16_t* out, int nthreads) {
  parallel_for(n, nthreads, [&](int64_t a, int64_t b) {
    for (int64_t i = a; i < b; ++i)
      out[i] = to_bf16(scale * normal_at(seed, stream, (uint64_t)(e0 + i)));
  });
}

// out[i] = fp32(mean + std * N_i).
void synth_normal_f32(uint64_t seed, uint32_t stream, int64_t e0, int64_t n,
                      double mean, double std_dev, float* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(mean + std_dev * normal_at(seed, stream, (uint64_t)(e0 + i)));
}

// out[i] = 2u - 1 with u uniform in (0, 1): one value per index.
void synth_uniform_pm1(uint64_t seed, uint32_t stream, int64_t e0, int64_t n,
                       double* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t o[4];
    block(seed, stream, 0, (uint64_t)(e0 + i), o);
    out[i] = 2.0 * unit(o[0], o[1]) - 1.0;
  }
}

// One 64-bit key per row, used to pick rows by sorting.
void synth_row_keys(uint64_t seed, uint32_t stream, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t o[4];
    block(seed, stream, 3, (uint64_t)i, o);
    out[i] = (((uint64_t)o[0]) << 32) | o[1];
  }
}

// Row-major [rows, H] tensor starting at global row t0:
//   out[t, i] = bf16(rho_t * x[t, i] + sqrt(1 - rho_t^2) * N_{t*H+i})
// with x given as bf16 bits (read exactly) and rho as fp64 per row.
void synth_correlated_bf16(uint64_t seed, uint32_t noise_stream,
                           const uint16_t* x, const double* rho, int64_t t0,
                           int64_t rows, int64_t H, uint16_t* out,
                           int nthreads) {
  parallel_for(rows * H, nthreads, [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) {
      int64_t t = j / H;
      uint32_t bits = ((uint32_t)x[j]) << 16;
      float xf;
      std::memcpy(&xf, &bits, 4);
      double r = rho[t];
      double n = normal_at(seed, noise_stream, (uint64_t)((t0 + t) * H + (j - t * H)));
      out[j] = to_bf16(r * (double)xf + std::sqrt(1.0 - r * r) * n);
    }
  });
}

// Row-major [rows, H] Student-t(3) tensor starting at global row t0; each
// row is scaled by row_scale[t] (e.g. 1, 1e3 or 0) before rounding.
void synth_student_t3_bf16(uint64_t seed, uint32_t stream, int64_t t0,
                           int64_t rows, int64_t H, const double* row_scale,
                           uint16_t* out, int nthreads) {
  parallel_for(rows * H, nthreads, [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) {
      int64_t t = j / H;
      double s = row_scale[t];
      if (s == 0.0) {
        out[j] = 0;
        continue;
      }
      uint64_t e = (uint64_t)((t0 + t) * H + (j - t * H));
      out[j] = to_bf16(s * student_t3_at(seed, stream, e));
    }
  });
}

}  // extern "C"
