// Host-side sanitizer program for the test infrastructure's C++: the fp64
// oracle, the comparison helpers, the N-gram hash oracle and the seeded input
// generator. Built with -fsanitize=address,undefined by
// tests/test_host_sanitizers.py and run on small inputs; any invalid access
// or undefined behaviour aborts the process.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
void synth_normal_bf16(uint64_t, uint32_t, int64_t, int64_t, double, uint16_t*, int);
void synth_normal_f32(uint64_t, uint32_t, int64_t, int64_t, double, double, float*);
void synth_uniform_pm1(uint64_t, uint32_t, int64_t, int64_t, double*);
void synth_row_keys(uint64_t, uint32_t, int64_t, uint64_t*);
void synth_correlated_bf16(uint64_t, uint32_t, const uint16_t*, const double*, int64_t, int64_t,
                           int64_t, uint16_t*, int);
void synth_student_t3_bf16(uint64_t, uint32_t, int64_t, int64_t, int64_t, const double*,
                           uint16_t*, int);
void synth_round_bf16(const double*, int64_t, uint16_t*);
void oracle_fwd_f64(const double*, const double*, const double*, const double*, const double*,
                    int64_t, int64_t, double, double*, double*, double*);
void oracle_bwd_f64(const double*, const double*, const double*, const double*, const double*,
                    const double*, int64_t, int64_t, double, double, double*, double*, double*,
                    double*, double*, double*);
void oracle_fwd_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const float*,
                     const float*, int64_t, int64_t, double, double*, double*, double*, int);
void oracle_bwd_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                     const float*, const float*, int64_t, int64_t, double, double, double*,
                     double*, double*, double*, double*, double*, int);
void oracle_round_bf16(const double*, int64_t, uint16_t*);
void oracle_compare_bf16(const uint16_t*, const double*, int64_t, int64_t, const uint8_t*,
                         double*, int);
void oracle_check_out(const uint16_t*, const double*, const uint16_t*, const uint16_t*,
                      const double*, int64_t, int64_t, double*, int);
void oracle_engram_hash(const int32_t*, int64_t, int64_t, int, int, const int32_t*,
                        const uint64_t*, const uint32_t*, uint32_t, int32_t*);
}

int main() {
  const int64_t T = 37, H = 72;
  const int64_t n = T * H;
  std::vector<uint16_t> x(n), k(n), v(n), g(n), kc(n), st(n);
  std::vector<float> wh(H), we(H);
  std::vector<double> rho(T), scale(T, 1.0);
  std::vector<uint64_t> keys(T);
  synth_normal_bf16(0, 1, 0, n, 1.0, x.data(), 3);
  synth_normal_bf16(0, 2, 0, n, 1.0, k.data(), 1);
  synth_normal_bf16(0, 3, 0, n, 1.0, v.data(), 4);
  synth_normal_bf16(0, 4, 0, n, 1.0, g.data(), 2);
  synth_normal_f32(0, 5, 0, H, 1.0, 0.1, wh.data());
  synth_normal_f32(0, 6, 0, H, 1.0, 0.1, we.data());
  synth_uniform_pm1(0, 7, 0, T, rho.data());
  synth_row_keys(0, 9, T, keys.data());
  synth_correlated_bf16(0, 8, x.data(), rho.data(), 5, T, H, kc.data(), 3);
  scale[3] = 0.0;
  scale[4] = 1e3;
  synth_student_t3_bf16(0, 1, 0, T, H, scale.data(), st.data(), 3);
  for (int i = 0; i < H; ++i) x[2 * H + i] = 0;            // a zero row

  std::vector<double> xd(n), kd(n), vd(n), gd(n), out(n), dx(n), dk(n), dv(n);
  for (int64_t i = 0; i < n; ++i) {
    xd[i] = (double)(int)(x[i] % 7) - 3.0;
    kd[i] = (double)(int)(k[i] % 5) - 2.0;
    vd[i] = (double)(int)(v[i] % 3) - 1.0;
    gd[i] = (double)(int)(g[i] % 9) - 4.0;
  }
  std::vector<double> whd(wh.begin(), wh.end()), wed(we.begin(), we.end());
  std::vector<double> gate(T), fst(T * 8), dwh(H), dwe(H), bst(T * 4), z(T), dd(T);
  oracle_fwd_f64(xd.data(), kd.data(), vd.data(), whd.data(), wed.data(), T, H, 1e-6,
                 out.data(), gate.data(), fst.data());
  oracle_bwd_f64(gd.data(), xd.data(), kd.data(), vd.data(), whd.data(), wed.data(), T, H,
                 1e-6, 1e-4, dx.data(), dk.data(), dv.data(), dwh.data(), dwe.data(),
                 bst.data());
  for (int th : {1, 3, 64}) {
    oracle_fwd_bf16(x.data(), kc.data(), v.data(), wh.data(), we.data(), T, H, 1e-6,
                    out.data(), gate.data(), z.data(), th);
    oracle_bwd_bf16(g.data(), x.data(), kc.data(), v.data(), wh.data(), we.data(), T, H,
                    1e-6, 1e-4, dx.data(), dk.data(), dv.data(), dwh.data(), dwe.data(),
                    dd.data(), th);
  }
  oracle_bwd_bf16(g.data(), x.data(), st.data(), v.data(), wh.data(), we.data(), T, H, 1e-6,
                  1e-4, nullptr, nullptr, nullptr, dwh.data(), dwe.data(), nullptr, 2);
  std::vector<uint16_t> rb(n), rb2(n);
  oracle_round_bf16(dx.data(), n, rb.data());
  synth_round_bf16(dx.data(), n, rb2.data());
  std::vector<uint8_t> cls(T, 0);
  cls[4] = 2;
  std::vector<double> acc(24, 0.0), res(4, 0.0);
  oracle_compare_bf16(rb.data(), dx.data(), T, H, cls.data(), acc.data(), 5);
  oracle_compare_bf16(rb.data(), dx.data(), T, H, nullptr, acc.data(), 1);
  oracle_check_out(rb.data(), dx.data(), x.data(), v.data(), gate.data(), T, H, res.data(), 4);

  const int L = 2, K = 3;
  std::vector<int32_t> tok(3 * 11), idx(3 * 11 * L * K), ngram = {2, 4};
  std::vector<uint64_t> mult(L * K * 4);
  std::vector<uint32_t> size(L * K);
  for (size_t i = 0; i < tok.size(); ++i) tok[i] = (int32_t)(keys[i % T] >> 33) - 7;
  for (size_t i = 0; i < mult.size(); ++i) mult[i] = keys[i % T] | 1u;
  for (size_t i = 0; i < size.size(); ++i) size[i] = 1u + (uint32_t)(keys[i] % 100000u);
  size[0] = 1;
  size[L * K - 1] = 2147483648u;
  oracle_engram_hash(tok.data(), 3, 11, L, K, ngram.data(), mult.data(), size.data(),
                     0xFFFFFFFFu, idx.data());
  for (size_t i = 0; i < idx.size(); ++i)
    if (idx[i] < 0) return 2;
  std::printf("host oracle program ok (%g %g)\n", acc[0], res[0]);
  return 0;
}
