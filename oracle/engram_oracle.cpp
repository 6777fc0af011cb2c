// Engram gate oracle: a plain, slow, fp64 CPU implementation.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
// call this file; it exists so that tests, the smoke check and the CPU
// baseline of the benchmark can check the GPU library against the definition.
// It shares no code with the GPU library.
//
// Source of the method: the zhichai.net TileKernels page ("DeepSeek 开源
// TileKernels ..."), section "5. Engram — 条件记忆门控", gate formula. In this
// file's notation, per token with rows x, k, v of width H:
//   a = RMSNorm of x with weight wh,   b = RMSNorm of k with weight we,
//   d = sum_i a_i b_i,   z = d / sqrt(H),   s = sign(z) sqrt|z|,
//   gate = 1 / (1 + exp(-s)),   out = x + gate * v.
// The same section names the fused forward/backward kernels and a separate
// weight-gradient reduction; the juejin.cn page (highlight 5) says the
// autograd wrapper covers forward, backward and weight-gradient reduction.
//
// Readings where the page is silent, each with its reason:
//   * hidden_states is the same row x that is normalised (the formula uses
//     both names for the one residual row);
//   * RMSNorm(x, w)_i = x_i / sqrt(mean(x^2) + eps) * w_i, eps inside the
//     root, eps = 1e-6 (the usual RMSNorm; the page gives no eps);
//   * sign(0) = 0, so a zero dot gives gate = 1/2 (the sign function's
//     usual value at 0);
//   * the derivative of signed_sqrt, 1 / (2 sqrt|z|), is evaluated as
//     1 / (2 sqrt(max(|z|, clamp))) so that it stays finite at z = 0, where
//     the true derivative is infinite (the clamp is a convention shared with
//     the GPU library, not a consequence of the formula);
//   * the backward is the chain rule of the forward, nothing else.
//
// Everything is fp64, row by row, with every intermediate of the formula
// materialised in the order the formula nests. Sums are sequential.
//
// Parity pins: see tests/test_oracle.py (closed forms, mirror and
// orthogonality cases, invariances, a library RMSNorm, finite differences
// and automatic differentiation of the forward). No function here is
// "parity unpinned" except the value of the clamp itself, which is a
// convention, not a consequence of the formula.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// Per-row quantities of the forward, in the formula's notation.
struct RowForward {
  double mean_sq_x;  // mean(x^2)
  double mean_sq_k;  // mean(k^2)
  double r_x;        // 1 / sqrt(mean(x^2) + eps)
  double r_k;        // 1 / sqrt(mean(k^2) + eps)
  double dot;        // d = dot(RMSNorm(x, wh), RMSNorm(k, we))
  double z;          // d * scalar, scalar = 1 / sqrt(H)
  double s;          // signed_sqrt(z)
  double gate;       // sigmoid(s)
};

double sign_of(double z) { return z > 0.0 ? 1.0 : (z < 0.0 ? -1.0 : 0.0); }

// RMSNorm of one row: out_i = row_i / sqrt(mean(row^2) + eps) * w_i.
// Returns mean(row^2) and 1 / sqrt(mean(row^2) + eps) through the pointers.
void rms_norm(const double* row, const double* w, int64_t H, double eps,
              double* out, double* mean_sq, double* r) {
  double sum_sq = 0.0;
  for (int64_t i = 0; i < H; ++i) sum_sq += row[i] * row[i];
  *mean_sq = sum_sq / (double)H;
  *r = 1.0 / std::sqrt(*mean_sq + eps);
  for (int64_t i = 0; i < H; ++i) out[i] = row[i] * (*r) * w[i];
}

// Forward of one token. a and b receive the two RMSNorm outputs.
RowForward forward_row(const double* x, const double* k, const double* wh,
                       const double* we, int64_t H, double eps, double* a,
                       double* b) {
  RowForward f;
  rms_norm(x, wh, H, eps, a, &f.mean_sq_x, &f.r_x);
  rms_norm(k, we, H, eps, b, &f.mean_sq_k, &f.r_k);
  double d = 0.0;
  for (int64_t i = 0; i < H; ++i) d += a[i] * b[i];
  f.dot = d;
  const double scalar = 1.0 / std::sqrt((double)H);
  f.z = d * scalar;
  f.s = sign_of(f.z) * std::sqrt(std::fabs(f.z));
  f.gate = 1.0 / (1.0 + std::exp(-f.s));
  return f;
}

// Per-row quantities of the backward.
struct RowBackward {
  double dgate;  // dL/dgate = sum_i gout_i * v_i
  double ds;     // dL/ds    = dgate * gate * (1 - gate)
  double dz;     // dL/dz    = ds / (2 sqrt(max(|z|, clamp)))
  double dd;     // dL/dd    = dz * scalar
};

// Backward of one token given its forward. Writes dx, dk, dv for the row and
// adds the row's contribution to dwh and dwe.
RowBackward backward_row(const double* gout, const double* x, const double* k,
                         const double* v, const double* wh, const double* we,
                         int64_t H, double clamp, const RowForward& f,
                         const double* a, const double* b, double* dx,
                         double* dk, double* dv, double* dwh, double* dwe) {
  RowBackward r;
  // output_i = x_i + gate * v_i
  double dg = 0.0;
  for (int64_t i = 0; i < H; ++i) dg += gout[i] * v[i];
  r.dgate = dg;
  for (int64_t i = 0; i < H; ++i) dv[i] = f.gate * gout[i];
  // gate = sigmoid(s): dgate/ds = gate (1 - gate). 1 - gate is sigmoid(-s),
  // evaluated as such: as 1 - gate it would keep only the rounding error of
  // gate where gate is close to 1 (|s| beyond about 15).
  r.ds = dg * f.gate * (1.0 / (1.0 + std::exp(f.s)));
  // s = sign(z) sqrt|z|: ds/dz = 1 / (2 sqrt|z|), |z| clamped from below
  r.dz = r.ds * 0.5 / std::sqrt(std::max(std::fabs(f.z), clamp));
  // z = d * scalar
  const double scalar = 1.0 / std::sqrt((double)H);
  r.dd = r.dz * scalar;
  // d = sum_i a_i b_i
  std::vector<double> da(H), db(H);
  for (int64_t i = 0; i < H; ++i) {
    da[i] = r.dd * b[i];
    db[i] = r.dd * a[i];
  }
  // a_i = x_i r_x wh_i with r_x = (mean(x^2) + eps)^(-1/2):
  //   da/dx: dx_j = r_x (wh_j da_j) - r_x^3 x_j / H * sum_i x_i wh_i da_i
  //   da/dwh: dwh_i += x_i r_x da_i
  double sx = 0.0, sk = 0.0;
  for (int64_t i = 0; i < H; ++i) {
    sx += x[i] * wh[i] * da[i];
    sk += k[i] * we[i] * db[i];
  }
  const double rx3 = f.r_x * f.r_x * f.r_x;
  const double rk3 = f.r_k * f.r_k * f.r_k;
  for (int64_t i = 0; i < H; ++i) {
    // the residual term of output_i = x_i + ... contributes gout_i
    dx[i] = gout[i] + f.r_x * wh[i] * da[i] - rx3 * x[i] * sx / (double)H;
    dk[i] = f.r_k * we[i] * db[i] - rk3 * k[i] * sk / (double)H;
    dwh[i] += x[i] * f.r_x * da[i];
    dwe[i] += k[i] * f.r_k * db[i];
  }
  return r;
}

double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

template <class F>
void run_threads(int64_t rows, int nthreads, F fn) {
  nthreads = std::max(1, (int)std::min<int64_t>(nthreads, std::max<int64_t>(rows, 1)));
  if (nthreads == 1) {
    fn(0, 0, rows);
    return;
  }
  std::vector<std::thread> pool;
  int64_t chunk = (rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = std::min(rows, (int64_t)t * chunk);
    int64_t hi = std::min(rows, lo + chunk);
    pool.emplace_back([=] { fn(t, lo, hi); });
  }
  for (auto& th : pool) th.join();
}

// Round fp64 values to bf16 bit patterns, to nearest with ties to even.
// The comparison convention for bf16 outputs is "the oracle's fp64 value,
// rounded once to bf16".
//
// Normal bf16 range: bf16 keeps the sign, the exponent and the top 7 stored
// significand bits of the value, so the fp64 significand (52 stored bits) is
// cut after its 7th bit and rounded on the 45 bits dropped. Elsewhere
// (subnormal bf16, overflow, zero, NaN) the value is rounded by scaling.
uint16_t round_one(double val) {
  uint64_t b;
  std::memcpy(&b, &val, 8);
  const uint64_t sign = b >> 63;
  const int exp_field = (int)((b >> 52) & 0x7FF);
  const int e = exp_field - 1023;                     // val = 1.f * 2^e
  if (exp_field != 0 && exp_field != 0x7FF && e >= -126 && e <= 127) {
    const uint64_t frac = b & ((1ull << 52) - 1);
    uint64_t keep = frac >> 45;                       // 7 stored bits
    const uint64_t dropped = frac & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    uint64_t biased = (uint64_t)(e + 127);
    if (dropped > half || (dropped == half && (keep & 1))) {
      ++keep;
      if (keep == 128) {                              // significand overflow
        keep = 0;
        ++biased;
      }
    }
    if (biased >= 255) return (uint16_t)((sign << 15) | 0x7F80);
    return (uint16_t)((sign << 15) | (biased << 7) | keep);
  }
  if (std::isnan(val)) return 0x7FC0;
  const uint16_t sbit = (uint16_t)(sign << 15);
  double mag = std::fabs(val);
  if (mag == 0.0) return sbit;
  if (e > 127) return sbit | 0x7F80;                  // beyond the bf16 range
  // |val| < 2^-126: bf16 subnormals are multiples of 2^-133.
  const double units = mag * 0x1p133;                 // exact scaling
  double lo = std::floor(units);
  const double frac = units - lo;
  if (frac > 0.5 || (frac == 0.5 && std::fmod(lo, 2.0) != 0.0)) lo += 1.0;
  // lo <= 2^7: 2^7 itself is the smallest normal 2^-126 (bits 0x0080).
  return sbit | (uint16_t)lo;
}

}  // namespace

extern "C" {

// Number of doubles written per row into `fwd_stats`:
// mean(x^2), mean(k^2), r_x, r_k, d, z, s, gate.
int oracle_fwd_stats_width(void) { return 8; }
// ... and into `bwd_stats`: dgate, ds, dz, dd.
int oracle_bwd_stats_width(void) { return 4; }

// Forward over T rows of fp64 inputs (row-major [T, H]).
// out [T, H], gate [T] and fwd_stats [T, 8] may each be null.
void oracle_fwd_f64(const double* x, const double* k, const double* v,
                    const double* wh, const double* we, int64_t T, int64_t H,
                    double eps, double* out, double* gate, double* fwd_stats) {
  std::vector<double> a(H), b(H);
  for (int64_t t = 0; t < T; ++t) {
    const double* xr = x + t * H;
    const double* kr = k + t * H;
    const double* vr = v + t * H;
    RowForward f = forward_row(xr, kr, wh, we, H, eps, a.data(), b.data());
    if (out)
      for (int64_t i = 0; i < H; ++i) out[t * H + i] = xr[i] + f.gate * vr[i];
    if (gate) gate[t] = f.gate;
    if (fwd_stats) {
      double* st = fwd_stats + t * 8;
      st[0] = f.mean_sq_x; st[1] = f.mean_sq_k; st[2] = f.r_x; st[3] = f.r_k;
      st[4] = f.dot; st[5] = f.z; st[6] = f.s; st[7] = f.gate;
    }
  }
}

// Backward over T rows of fp64 inputs. dx, dk, dv are [T, H]; dwh and dwe
// [H] are overwritten with the sums over the T rows; bwd_stats [T, 4] may be
// null.
void oracle_bwd_f64(const double* gout, const double* x, const double* k,
                    const double* v, const double* wh, const double* we,
                    int64_t T, int64_t H, double eps, double clamp, double* dx,
                    double* dk, double* dv, double* dwh, double* dwe,
                    double* bwd_stats) {
  std::vector<double> a(H), b(H);
  for (int64_t i = 0; i < H; ++i) dwh[i] = dwe[i] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t o = t * H;
    RowForward f = forward_row(x + o, k + o, wh, we, H, eps, a.data(), b.data());
    RowBackward r = backward_row(gout + o, x + o, k + o, v + o, wh, we, H, clamp,
                                 f, a.data(), b.data(), dx + o, dk + o, dv + o,
                                 dwh, dwe);
    if (bwd_stats) {
      double* st = bwd_stats + t * 4;
      st[0] = r.dgate; st[1] = r.ds; st[2] = r.dz; st[3] = r.dd;
    }
  }
}

// Forward over `rows` rows of bf16 inputs (uint16 bit patterns, row-major)
// and fp32 weights, every value widened exactly to fp64 first. Rows are split
// over `nthreads` threads in contiguous chunks. out [rows, H], gate [rows],
// z [rows] may each be null.
void oracle_fwd_bf16(const uint16_t* x, const uint16_t* k, const uint16_t* v,
                     const float* wh, const float* we, int64_t rows, int64_t H,
                     double eps, double* out, double* gate, double* z,
                     int nthreads) {
  std::vector<double> whd(wh, wh + H), wed(we, we + H);
  run_threads(rows, nthreads, [&](int, int64_t lo, int64_t hi) {
    std::vector<double> xr(H), kr(H), vr(H), a(H), b(H);
    for (int64_t t = lo; t < hi; ++t) {
      for (int64_t i = 0; i < H; ++i) {
        xr[i] = bf16_bits_to_double(x[t * H + i]);
        kr[i] = bf16_bits_to_double(k[t * H + i]);
        vr[i] = bf16_bits_to_double(v[t * H + i]);
      }
      RowForward f = forward_row(xr.data(), kr.data(), whd.data(), wed.data(), H,
                                 eps, a.data(), b.data());
      if (out)
        for (int64_t i = 0; i < H; ++i) out[t * H + i] = xr[i] + f.gate * vr[i];
      if (gate) gate[t] = f.gate;
      if (z) z[t] = f.z;
    }
  });
}

// Backward over `rows` rows of bf16 inputs. dx, dk, dv [rows, H] may be null
// (then only the weight gradients and per-row scalars are produced); dwh and
// dwe [H] are overwritten with the fp64 sums over these rows (per-thread
// partials added in thread order); dd [rows] may be null.
void oracle_bwd_bf16(const uint16_t* gout, const uint16_t* x, const uint16_t* k,
                     const uint16_t* v, const float* wh, const float* we,
                     int64_t rows, int64_t H, double eps, double clamp,
                     double* dx, double* dk, double* dv, double* dwh,
                     double* dwe, double* dd, int nthreads) {
  std::vector<double> whd(wh, wh + H), wed(we, we + H);
  nthreads = std::max(1, (int)std::min<int64_t>(nthreads, std::max<int64_t>(rows, 1)));
  std::vector<std::vector<double>> pwh(nthreads, std::vector<double>(H, 0.0));
  std::vector<std::vector<double>> pwe(nthreads, std::vector<double>(H, 0.0));
  run_threads(rows, nthreads, [&](int tid, int64_t lo, int64_t hi) {
    std::vector<double> gr(H), xr(H), kr(H), vr(H), a(H), b(H);
    std::vector<double> tx(H), tk(H), tv(H);
    for (int64_t t = lo; t < hi; ++t) {
      for (int64_t i = 0; i < H; ++i) {
        gr[i] = bf16_bits_to_double(gout[t * H + i]);
        xr[i] = bf16_bits_to_double(x[t * H + i]);
        kr[i] = bf16_bits_to_double(k[t * H + i]);
        vr[i] = bf16_bits_to_double(v[t * H + i]);
      }
      RowForward f = forward_row(xr.data(), kr.data(), whd.data(), wed.data(), H,
                                 eps, a.data(), b.data());
      RowBackward r = backward_row(gr.data(), xr.data(), kr.data(), vr.data(),
                                   whd.data(), wed.data(), H, clamp, f, a.data(),
                                   b.data(), tx.data(), tk.data(), tv.data(),
                                   pwh[tid].data(), pwe[tid].data());
      if (dx) std::memcpy(dx + t * H, tx.data(), H * sizeof(double));
      if (dk) std::memcpy(dk + t * H, tk.data(), H * sizeof(double));
      if (dv) std::memcpy(dv + t * H, tv.data(), H * sizeof(double));
      if (dd) dd[t] = r.dd;
    }
  });
  for (int64_t i = 0; i < H; ++i) {
    double sh = 0.0, se = 0.0;
    for (int t = 0; t < nthreads; ++t) {
      sh += pwh[t][i];
      se += pwe[t][i];
    }
    dwh[i] = sh;
    dwe[i] = se;
  }
}

void oracle_round_bf16(const double* v, int64_t n, uint16_t* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = round_one(v[j]);
}

}  // extern "C"
