// Host-side sanitizer program for the C ABI of include/tk_engram.h: every
// argument check of every entry point, run without a GPU (each call below
// returns its status before any device work). Built from the library
// sources with the host half under -fsanitize=address,undefined by
// tests/test_host_sanitizers.py.

#include <cstdint>
#include <cstdio>

#include "tk_engram.h"

#define EXPECT(call, want)                                                     \
  do {                                                                         \
    const tk_status got_ = (call);                                             \
    if (got_ != (want)) {                                                      \
      std::printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                  (int)got_, (int)(want));                                     \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main() {
  // 16-byte aligned fake device addresses: never dereferenced by the checks
  uint16_t* a = reinterpret_cast<uint16_t*>(uintptr_t(0x10000));
  float* f = reinterpret_cast<float*>(uintptr_t(0x10000));
  float* f4 = reinterpret_cast<float*>(uintptr_t(0x10004));
  double* d = reinterpret_cast<double*>(uintptr_t(0x10000));
  int32_t* i32 = reinterpret_cast<int32_t*>(uintptr_t(0x10000));

  for (int s = -1; s < 10; ++s)
    if (!tk_status_string(s)) return 1;
  if (tk_abi_version() != TK_ENGRAM_ABI_VERSION) return 1;
  const int64_t Ts[] = {0, 1, 7, 1000, 65537, (int64_t)1 << 40};
  const int64_t Hs[] = {-8, 0, 8, 12, 256, 4096, 7168, 8192, 8200};
  for (int64_t T : Ts)
    for (int64_t H : Hs) {
      const int64_t P = tk_engram_num_partials(T, H);
      if (P < 0 || P > 256) return 1;
      if (tk_engram_bwd_workspace_bytes(T, H) != (size_t)P * (size_t)(H > 0 ? H : 0) * 4 &&
          P != 0)
        return 1;
    }

  EXPECT(tk_engram_gate_fwd(a, a, a, f, f, a, f, -1, 64, 1e-6, nullptr), TK_ERR_SHAPE);
  EXPECT(tk_engram_gate_fwd(a, a, a, f, f, a, f, 4, 12, 1e-6, nullptr), TK_ERR_ALIGN);
  EXPECT(tk_engram_gate_fwd(a, a, a, f, f, a, f, 4, 8200, 1e-6, nullptr), TK_ERR_UNSUPPORTED);
  EXPECT(tk_engram_gate_fwd(a, a, a, f, f, a, f, 4, 64, 0.0, nullptr), TK_ERR_VALUE);
  EXPECT(tk_engram_gate_fwd(a, a, a, f, f, a, f, 4, 64, 1e-39, nullptr), TK_ERR_VALUE);
  EXPECT(tk_engram_gate_fwd(nullptr, a, a, f, f, a, f, 0, 64, 0x1p-126, nullptr), TK_SUCCESS);
  EXPECT(tk_engram_gate_fwd(nullptr, a, a, f, f, a, f, 0, 64, 1e-6, nullptr), TK_SUCCESS);
  EXPECT(tk_engram_gate_fwd(a, nullptr, a, f, f, a, f, 4, 64, 1e-6, nullptr), TK_ERR_NULL);
  EXPECT(tk_engram_gate_fwd(a, a, a, f4, f, a, f, 4, 64, 1e-6, nullptr), TK_ERR_ALIGN);

  EXPECT(tk_engram_gate_bwd(a, a, a, a, f, f, a, a, a, f, 1 << 30, 4, 64, 1e-6, 0.0, nullptr),
         TK_ERR_VALUE);
  EXPECT(tk_engram_gate_bwd(a, a, a, a, f, f, a, a, a, f, 4, 4, 64, 1e-6, 1e-4, nullptr),
         TK_ERR_WORKSPACE);
  EXPECT(tk_engram_gate_bwd(a, a, a, a, f, f, a, a, a, nullptr, 1 << 30, 4, 64, 1e-6, 1e-4,
                            nullptr),
         TK_ERR_NULL);
  for (double clamp : {1e-39, 1e-300, 1e39})
    EXPECT(tk_engram_gate_bwd(a, a, a, a, f, f, a, a, a, f, 1 << 30, 4, 64, 1e-6, clamp, nullptr),
           TK_ERR_VALUE);

  // the fused-weight forms: w (fp64) in place of wh and we
  EXPECT(tk_engram_gate_fwd_fused(a, a, a, d, a, f, -1, 64, 1e-6, nullptr), TK_ERR_SHAPE);
  EXPECT(tk_engram_gate_fwd_fused(a, a, a, nullptr, a, f, 4, 64, 1e-6, nullptr), TK_ERR_NULL);
  EXPECT(tk_engram_gate_fwd_fused(a, a, a, d + 1, a, f, 4, 64, 1e-6, nullptr), TK_ERR_ALIGN);
  EXPECT(tk_engram_gate_fwd_fused(nullptr, a, a, nullptr, a, f, 0, 64, 1e-6, nullptr), TK_SUCCESS);
  EXPECT(tk_engram_gate_bwd_fused(a, a, a, a, d, a, a, a, f, 4, 4, 64, 1e-6, 1e-4, nullptr),
         TK_ERR_WORKSPACE);
  EXPECT(tk_engram_gate_bwd_fused(a, a, a, a, nullptr, a, a, a, f, 1 << 30, 4, 64, 1e-6, 1e-4,
                                  nullptr),
         TK_ERR_NULL);
  EXPECT(tk_engram_gate_bwd_fused(a, a, a, a, d, a, a, a, f, 1 << 30, 4, 64, 1e-6, 0.0, nullptr),
         TK_ERR_VALUE);

  // the allocation-free backward: failing checks only (a passing call would launch)
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, f, f, a, a, a, f, f, -1, 64, 1e-6, 1e-4,
                                           nullptr),
         TK_ERR_SHAPE);
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, f, f, a, a, a, nullptr, f, 4, 64, 1e-6,
                                           1e-4, nullptr),
         TK_ERR_NULL);
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, f, f, a, a, a, f, f4, 4, 64, 1e-6, 1e-4,
                                           nullptr),
         TK_ERR_ALIGN);
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, f, f, a, a, a, f, f, 4, 64, 1e-6, 0.0,
                                           nullptr),
         TK_ERR_VALUE);
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, nullptr, f, a, a, a, f, f, 0, 64, 1e-6,
                                           1e-4, nullptr),
         TK_ERR_NULL);
  EXPECT(tk_engram_gate_bwd_reduce_noalloc(a, a, a, a, f, f4, a, a, a, f, f, 0, 64, 1e-6, 1e-4,
                                           nullptr),
         TK_ERR_ALIGN);

  // launches per call: a pure function of (T, H), 0 exactly when there are no partials
  for (int64_t T : Ts)
    for (int64_t H : Hs)
      for (int32_t b = 0; b < 2; ++b) {
        const int64_t L = tk_engram_gate_launches(T, H, b);
        if (L < 0 || (L == 0) != (tk_engram_num_partials(T, H) == 0)) return 1;
      }

  EXPECT(tk_engram_grad_w_reduce(f, TK_ENGRAM_MAX_PARTIALS + 1, 64, f, f, f, f, nullptr),
         TK_ERR_UNSUPPORTED);
  EXPECT(tk_engram_grad_w_reduce(f, -1, 64, f, f, f, f, nullptr), TK_ERR_SHAPE);
  EXPECT(tk_engram_grad_w_reduce(f, 3, 64, f, f, f4, f, nullptr), TK_ERR_ALIGN);
  EXPECT(tk_engram_fused_weight(f, f, d, -1, nullptr), TK_ERR_SHAPE);
  EXPECT(tk_engram_fused_weight(f, f, nullptr, 8, nullptr), TK_ERR_NULL);

  const int32_t ngram[2] = {2, 3}, bad_ngram[2] = {2, 5};
  uint64_t mult[2 * 8 * 4] = {};
  uint32_t sizes[16];
  for (int i = 0; i < 16; ++i) sizes[i] = 1021;
  EXPECT(tk_engram_hash(i32, 2, 5, 2, 8, bad_ngram, mult, sizes, 0, i32, nullptr), TK_ERR_VALUE);
  EXPECT(tk_engram_hash(i32, 2, 5, 2, 17, ngram, mult, sizes, 0, i32, nullptr),
         TK_ERR_UNSUPPORTED);
  EXPECT(tk_engram_hash(i32, 0, 5, 2, 8, ngram, mult, sizes, 0, nullptr, nullptr), TK_SUCCESS);
  sizes[15] = 0;
  EXPECT(tk_engram_hash(i32, 2, 5, 2, 8, ngram, mult, sizes, 0, i32, nullptr), TK_ERR_VALUE);

  const int64_t off[2] = {0, 50};
  const uint32_t rows[2] = {50, 51};
  EXPECT(tk_engram_gather(i32, 4, 2, a, 100, 64, off, rows, a, nullptr), TK_ERR_VALUE);
  EXPECT(tk_engram_gather(i32, 4, 2, a, 100, 12, off, rows, a, nullptr), TK_ERR_ALIGN);
  EXPECT(tk_engram_gather(i32, 4, 33, a, 100, 64, off, rows, a, nullptr), TK_ERR_UNSUPPORTED);

  const void* srcs[2] = {a, a};
  void* dsts[5] = {a, a, a, a, a};
  EXPECT(tk_engram_stream_probe(srcs, 2, dsts, 5, 64, nullptr), TK_ERR_SHAPE);
  EXPECT(tk_engram_stream_probe(srcs, 2, dsts, 2, 40, nullptr), TK_ERR_ALIGN);
  EXPECT(tk_engram_copy_probe(a, a, 40, nullptr), TK_ERR_ALIGN);
  std::printf("host ABI program ok\n");
  return 0;
}
