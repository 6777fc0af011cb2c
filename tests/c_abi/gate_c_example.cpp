// The Engram gate library used from plain host C++ through include/tk_engram.h
// and the HIP runtime alone (no Python, no torch): a forward, backward and
// weight-gradient reduction on a small batch, checked against properties the
// gate formula fixes exactly (zhichai.net TileKernels page, section "5. Engram").
//
//   row 0: x and k on disjoint halves of the hidden axis -> the dot is 0,
//          gate = sigmoid(0) = 1/2 exactly and out = bf16(x + v / 2)
//   all rows: gate in (0, 1); dv = bf16(gate * grad_out) bit for bit
//   reruns: dwh and dwe bit-identical
//   the fused-weight forward and backward (w = wh * we from
//   tk_engram_fused_weight) and the allocation-free backward + reduction:
//   the plain calls' outputs bit for bit
// Exits 0 and prints "c abi example ok" on success.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "tk_engram.h"

#define HIP_OK(x)                                                        \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      std::printf("%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 1;                                                          \
    }                                                                    \
  } while (0)

#define TK_OK(x)                                                         \
  do {                                                                   \
    tk_status s_ = (x);                                                  \
    if (s_ != TK_SUCCESS) {                                              \
      std::printf("%s failed: %s\n", #x, tk_status_string(s_));          \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static uint16_t to_bf16(float f) {  // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int main() {
  const int64_t T = 9, H = 7168;
  const size_t n = (size_t)(T * H);
  std::vector<uint16_t> x(n), k(n), v(n), g(n);
  std::vector<float> wh(H), we(H);
  uint32_t s = 12345u;
  auto next = [&]() {  // xorshift32 in [-1, 1)
    s ^= s << 13; s ^= s >> 17; s ^= s << 5;
    return (float)(s >> 8) / (float)(1u << 23) - 1.0f;
  };
  for (size_t i = 0; i < n; ++i) {
    x[i] = to_bf16(next());
    k[i] = to_bf16(next());
    v[i] = to_bf16(next());
    g[i] = to_bf16(next());
  }
  for (int64_t i = 0; i < H; ++i) {
    wh[i] = 1.0f + 0.1f * next();
    we[i] = 1.0f + 0.1f * next();
  }
  for (int64_t i = 0; i < H; ++i) {  // row 0: disjoint supports
    if (i < H / 2) k[i] = 0; else x[i] = 0;
  }

  const int64_t P = tk_engram_num_partials(T, H);
  const size_t ws_bytes = tk_engram_bwd_workspace_bytes(T, H);
  uint16_t *dx_, *dk_, *dv_, *dout, *dxg, *dkg, *dvg, *dgo;
  float *dwh_, *dwe_, *dgate, *dws, *dgwh, *dgwe;
  HIP_OK(hipMalloc(&dx_, n * 2));
  HIP_OK(hipMalloc(&dk_, n * 2));
  HIP_OK(hipMalloc(&dv_, n * 2));
  HIP_OK(hipMalloc(&dgo, n * 2));
  HIP_OK(hipMalloc(&dout, n * 2));
  HIP_OK(hipMalloc(&dxg, n * 2));
  HIP_OK(hipMalloc(&dkg, n * 2));
  HIP_OK(hipMalloc(&dvg, n * 2));
  HIP_OK(hipMalloc(&dwh_, H * 4));
  HIP_OK(hipMalloc(&dwe_, H * 4));
  HIP_OK(hipMalloc(&dgate, T * 4));
  HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMalloc(&dgwh, H * 4));
  HIP_OK(hipMalloc(&dgwe, H * 4));
  HIP_OK(hipMemcpy(dx_, x.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk_, k.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv_, v.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dgo, g.data(), n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dwh_, wh.data(), H * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dwe_, we.data(), H * 4, hipMemcpyHostToDevice));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  std::vector<float> gwh[2], gwe[2];
  for (int rep = 0; rep < 2; ++rep) {
    TK_OK(tk_engram_gate_fwd(dx_, dk_, dv_, dwh_, dwe_, dout, dgate, T, H, 1e-6, st));
    TK_OK(tk_engram_gate_bwd(dgo, dx_, dk_, dv_, dwh_, dwe_, dxg, dkg, dvg, dws, ws_bytes, T, H,
                             1e-6, 1e-4, st));
    TK_OK(tk_engram_grad_w_reduce(dws, P, H, dwh_, dwe_, dgwh, dgwe, st));
    HIP_OK(hipStreamSynchronize(st));
    gwh[rep].resize(H);
    gwe[rep].resize(H);
    HIP_OK(hipMemcpy(gwh[rep].data(), dgwh, H * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gwe[rep].data(), dgwe, H * 4, hipMemcpyDeviceToHost));
  }
  std::vector<uint16_t> out(n), dv(n);
  std::vector<float> gate(T);
  HIP_OK(hipMemcpy(out.data(), dout, n * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dv.data(), dvg, n * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(gate.data(), dgate, T * 4, hipMemcpyDeviceToHost));

  if (gate[0] != 0.5f) { std::printf("row 0 gate %.9g != 0.5\n", gate[0]); return 1; }
  for (int64_t i = 0; i < H; ++i) {
    const uint16_t want = to_bf16(from_bf16(x[i]) + 0.5f * from_bf16(v[i]));
    if (out[i] != want) { std::printf("row 0 out[%lld] differs\n", (long long)i); return 1; }
  }
  for (int64_t t = 0; t < T; ++t) {
    if (!(gate[t] > 0.0f && gate[t] < 1.0f)) { std::printf("gate[%lld] out of (0,1)\n", (long long)t); return 1; }
    for (int64_t i = 0; i < H; ++i) {
      const size_t j = (size_t)(t * H + i);
      if (dv[j] != to_bf16(gate[t] * from_bf16(g[j]))) {
        std::printf("dv[%lld][%lld] differs\n", (long long)t, (long long)i);
        return 1;
      }
    }
  }
  if (std::memcmp(gwh[0].data(), gwh[1].data(), H * 4) || std::memcmp(gwe[0].data(), gwe[1].data(), H * 4)) {
    std::printf("weight gradients differ between reruns\n");
    return 1;
  }

  // the same step through the fused weight and through the allocation-free
  // backward, into fresh outputs: every byte must match the plain calls
  double* dw;
  uint16_t *fout, *fdx, *fdk, *fdv, *ndx, *ndk, *ndv;
  float *fgate, *fws, *ndwh, *ndwe;
  HIP_OK(hipMalloc(&dw, H * 8));
  HIP_OK(hipMalloc(&fout, n * 2));
  HIP_OK(hipMalloc(&fdx, n * 2));
  HIP_OK(hipMalloc(&fdk, n * 2));
  HIP_OK(hipMalloc(&fdv, n * 2));
  HIP_OK(hipMalloc(&ndx, n * 2));
  HIP_OK(hipMalloc(&ndk, n * 2));
  HIP_OK(hipMalloc(&ndv, n * 2));
  HIP_OK(hipMalloc(&fgate, T * 4));
  HIP_OK(hipMalloc(&fws, ws_bytes));
  HIP_OK(hipMalloc(&ndwh, H * 4));
  HIP_OK(hipMalloc(&ndwe, H * 4));
  TK_OK(tk_engram_fused_weight(dwh_, dwe_, dw, H, st));
  TK_OK(tk_engram_gate_fwd_fused(dx_, dk_, dv_, dw, fout, fgate, T, H, 1e-6, st));
  TK_OK(tk_engram_gate_bwd_fused(dgo, dx_, dk_, dv_, dw, fdx, fdk, fdv, fws, ws_bytes, T, H, 1e-6,
                                 1e-4, st));
  TK_OK(tk_engram_gate_bwd_reduce_noalloc(dgo, dx_, dk_, dv_, dwh_, dwe_, ndx, ndk, ndv, ndwh, ndwe,
                                          T, H, 1e-6, 1e-4, st));
  HIP_OK(hipStreamSynchronize(st));
  struct Pair { const void* a; const void* b; size_t bytes; const char* name; };
  const Pair pairs[] = {{dout, fout, n * 2, "fused out"}, {dgate, fgate, (size_t)T * 4, "fused gate"},
                        {dxg, fdx, n * 2, "fused dx"},   {dkg, fdk, n * 2, "fused dk"},
                        {dvg, fdv, n * 2, "fused dv"},   {dws, fws, ws_bytes, "fused partials"},
                        {dxg, ndx, n * 2, "no-alloc dx"}, {dkg, ndk, n * 2, "no-alloc dk"},
                        {dvg, ndv, n * 2, "no-alloc dv"}, {dgwh, ndwh, (size_t)H * 4, "no-alloc dwh"},
                        {dgwe, ndwe, (size_t)H * 4, "no-alloc dwe"}};
  for (const Pair& p : pairs) {
    std::vector<uint8_t> ha(p.bytes), hb(p.bytes);
    HIP_OK(hipMemcpy(ha.data(), p.a, p.bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hb.data(), p.b, p.bytes, hipMemcpyDeviceToHost));
    if (std::memcmp(ha.data(), hb.data(), p.bytes)) {
      std::printf("%s differs from the plain calls\n", p.name);
      return 1;
    }
  }
  for (void* p : {(void*)dw, (void*)fout, (void*)fdx, (void*)fdk, (void*)fdv, (void*)ndx,
                  (void*)ndk, (void*)ndv, (void*)fgate, (void*)fws, (void*)ndwh, (void*)ndwe})
    HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(st));
  for (void* p : {(void*)dx_, (void*)dk_, (void*)dv_, (void*)dgo, (void*)dout, (void*)dxg,
                  (void*)dkg, (void*)dvg, (void*)dwh_, (void*)dwe_, (void*)dgate, (void*)dws,
                  (void*)dgwh, (void*)dgwe})
    HIP_OK(hipFree(p));
  std::printf("c abi example ok: T=%lld H=%lld P=%lld gate[1]=%.6f\n", (long long)T,
              (long long)H, (long long)P, gate[1]);
  return 0;
}
