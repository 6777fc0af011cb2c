// N-gram hash of the Engram memory (zhichai.net TileKernels page, section
// "5. Engram": engram_hash) for AMD MI355X (gfx950), and its C ABI entry
// point tk_engram_hash declared in include/tk_engram.h.
//
// For every token position s of every sequence b, and every table j of
// every N-gram layer l:
//   h   = XOR over i < n_l of ( tok(b, s - i) * a[l][j][i]  mod 2^64 )
//   idx = h mod M[l][j]
// where tok(b, p) is the token id as an unsigned 32-bit pattern, or `pad`
// for p < 0. The multipliers a and table sizes M are the caller's.
//
// One thread per token. The few multipliers, sizes and precomputed Barrett
// reciprocals travel by value in the kernel arguments (scalar registers).
// The N-gram window of a token is re-read by its neighbours' threads, so
// the token loads hit in cache; the kernel streams 4 bytes in and 4 * L * K
// bytes out per token. h mod M is computed exactly with a Barrett quotient
// q = mulhi64(h, floor((2^64 - 1) / M)), which is at most 2 below
// floor(h / M), followed by two conditional subtractions.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tk_engram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTables = TK_ENGRAM_HASH_MAX_TABLES;  // L * K
constexpr int kMaxN = TK_ENGRAM_HASH_MAX_NGRAM;
constexpr int kHashBlock = 256;

struct HashParams {
  uint64_t mult[kMaxTables][kMaxN];
  uint64_t recip[kMaxTables];  // floor((2^64 - 1) / M)
  uint32_t mod[kMaxTables];    // M
  int32_t n[kMaxTables];       // N-gram order of the table's layer
  int32_t tables;              // L * K
  uint32_t pad;
};

__device__ __forceinline__ uint32_t mod_exact(uint64_t h, uint64_t recip, uint32_t m) {
  const uint64_t q = __umul64hi(h, recip);
  uint64_t r = h - q * (uint64_t)m;
  r = r >= m ? r - m : r;
  r = r >= m ? r - m : r;
  return (uint32_t)r;
}

__device__ __forceinline__ uint32_t table_index(const uint32_t (&tok)[kMaxN],
                                                const HashParams& p, int q) {
  uint64_t h = 0;
#pragma unroll
  for (int i = 0; i < kMaxN; ++i)
    if (i < p.n[q]) h ^= (uint64_t)tok[i] * p.mult[q][i];
  return mod_exact(h, p.recip[q], p.mod[q]);
}

__device__ __forceinline__ void window(const int32_t* __restrict__ seq, int64_t s,
                                       uint32_t pad, uint32_t (&tok)[kMaxN]) {
#pragma unroll
  for (int i = 0; i < kMaxN; ++i) tok[i] = s - i >= 0 ? (uint32_t)seq[s - i] : pad;
}

// L * K == LK, a multiple of 4: each token's indices leave in 16-byte stores.
template <int LK>
__global__ __launch_bounds__(kHashBlock) void hash_kernel_vec(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    u32x4* __restrict__ out) {
  const int64_t s = (int64_t)blockIdx.x * kHashBlock + threadIdx.x;
  if (s >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[kMaxN];
  window(tokens + b * S, s, p.pad, tok);
  u32x4* o = out + (b * S + s) * (LK / 4);
#pragma unroll
  for (int q4 = 0; q4 < LK / 4; ++q4) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = table_index(tok, p, 4 * q4 + e);
    o[q4] = v;
  }
}

// Any L * K: one 4-byte store per index.
__global__ __launch_bounds__(kHashBlock) void hash_kernel_any(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    uint32_t* __restrict__ out) {
  const int64_t s = (int64_t)blockIdx.x * kHashBlock + threadIdx.x;
  if (s >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[kMaxN];
  window(tokens + b * S, s, p.pad, tok);
  uint32_t* o = out + (b * S + s) * p.tables;
  for (int q = 0; q < p.tables; ++q) o[q] = table_index(tok, p, q);
}

template <int LK>
hipError_t launch_vec(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                      dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(hash_kernel_vec<LK>, grid, dim3(kHashBlock), 0, st, tokens, S, p,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace

extern "C" tk_status tk_engram_hash(const int32_t* tokens, int64_t B, int64_t S,
                                    int32_t L, int32_t K, const int32_t* ngram,
                                    const uint64_t* mult, const uint32_t* table_size,
                                    uint32_t pad, int32_t* out, void* stream) {
  if (B < 0 || S < 0 || L < 1 || K < 1) return TK_ERR_SHAPE;
  if ((int64_t)L * K > kMaxTables || B > TK_ENGRAM_HASH_MAX_BATCH) return TK_ERR_UNSUPPORTED;
  if (!ngram || !mult || !table_size) return TK_ERR_NULL;
  for (int l = 0; l < L; ++l)
    if (ngram[l] < 1 || ngram[l] > kMaxN) return TK_ERR_VALUE;
  for (int q = 0; q < L * K; ++q)
    if (table_size[q] < 1 || table_size[q] > TK_ENGRAM_HASH_MAX_TABLE_SIZE) return TK_ERR_VALUE;
  if (B == 0 || S == 0) return TK_SUCCESS;
  if (!tokens || !out) return TK_ERR_NULL;
  if (((uintptr_t)tokens & 3u) || ((uintptr_t)out & 15u)) return TK_ERR_ALIGN;

  HashParams p = {};
  p.tables = L * K;
  p.pad = pad;
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < K; ++j) {
      const int q = l * K + j;
      for (int i = 0; i < kMaxN; ++i) p.mult[q][i] = mult[(int64_t)q * kMaxN + i];
      p.mod[q] = table_size[q];
      p.recip[q] = UINT64_MAX / table_size[q];
      p.n[q] = ngram[l];
    }
  const dim3 grid((unsigned)((S + kHashBlock - 1) / kHashBlock), (unsigned)B);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (p.tables) {
    case 4: e = launch_vec<4>(tokens, S, p, out, grid, st); break;
    case 8: e = launch_vec<8>(tokens, S, p, out, grid, st); break;
    case 12: e = launch_vec<12>(tokens, S, p, out, grid, st); break;
    case 16: e = launch_vec<16>(tokens, S, p, out, grid, st); break;
    case 20: e = launch_vec<20>(tokens, S, p, out, grid, st); break;
    case 24: e = launch_vec<24>(tokens, S, p, out, grid, st); break;
    case 28: e = launch_vec<28>(tokens, S, p, out, grid, st); break;
    case 32: e = launch_vec<32>(tokens, S, p, out, grid, st); break;
    default:
      hipLaunchKernelGGL(hash_kernel_any, grid, dim3(kHashBlock), 0, st, tokens, S, p,
                         reinterpret_cast<uint32_t*>(out));
      e = hipGetLastError();
  }
  return e == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}
