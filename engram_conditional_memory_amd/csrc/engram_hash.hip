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
// reciprocals travel by value in the kernel arguments, one contiguous record
// per table. The N-gram window of a token is re-read by its neighbours'
// threads, so the token loads hit in cache; the kernel streams 4 bytes in and
// 4 * L * K bytes out per token. h mod M is computed exactly with a Barrett
// quotient q = mulhi64(h, floor((2^64 - 1) / M)), which is at most 2 below
// floor(h / M), followed by two conditional subtractions.
//
// Every table runs the same number of products, NMAX (the largest N of any
// layer), with the multipliers of positions i >= N set to 0 on the host: a
// product with 0 leaves the XOR unchanged, so the result is the N-gram hash
// of the table's own layer, and the kernel has no branches on N. Branching on
// a table's N made each wave wait for that table's parameters from the
// scalar cache before it could go on, which cost a third of the throughput.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tk_engram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTables = TK_ENGRAM_HASH_MAX_TABLES;  // L * K
constexpr int kMaxN = TK_ENGRAM_HASH_MAX_NGRAM;
constexpr int kHashBlock = 256;

struct TableParams {
  uint64_t mult[kMaxN];  // multiplier of window position i; 0 for i >= N
  uint64_t recip;        // floor((2^64 - 1) / M)
  uint32_t mod;          // M
  uint32_t unused;
};

struct HashParams {
  TableParams t[kMaxTables];
  int32_t tables;  // L * K
  uint32_t pad;
};

__device__ __forceinline__ uint32_t mod_exact(uint64_t h, uint64_t recip, uint32_t m) {
  const uint64_t q = __umul64hi(h, recip);
  uint64_t r = h - q * (uint64_t)m;
  r = r >= m ? r - m : r;
  r = r >= m ? r - m : r;
  return (uint32_t)r;
}

template <int NMAX>
__device__ __forceinline__ uint32_t table_index(const uint32_t (&tok)[NMAX],
                                                const TableParams& t) {
  uint64_t h = 0;
#pragma unroll
  for (int i = 0; i < NMAX; ++i) h ^= (uint64_t)tok[i] * t.mult[i];
  return mod_exact(h, t.recip, t.mod);
}

// tok[i] = token at position s - i of the sequence, `pad` before its start.
template <int NMAX>
__device__ __forceinline__ void window(const int32_t* __restrict__ seq, int64_t s,
                                       uint32_t pad, uint32_t (&tok)[NMAX]) {
#pragma unroll
  for (int i = 0; i < NMAX; ++i) tok[i] = s - i >= 0 ? (uint32_t)seq[s - i] : pad;
}

// L * K == LK, a multiple of 4: each token's indices leave in 16-byte stores.
template <int LK, int NMAX>
__global__ __launch_bounds__(kHashBlock) void hash_kernel_vec(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    u32x4* __restrict__ out) {
  const int64_t s = (int64_t)blockIdx.x * kHashBlock + threadIdx.x;
  if (s >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[NMAX];
  window<NMAX>(tokens + b * S, s, p.pad, tok);
  u32x4* o = out + (b * S + s) * (LK / 4);
#pragma unroll
  for (int q4 = 0; q4 < LK / 4; ++q4) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = table_index<NMAX>(tok, p.t[4 * q4 + e]);
    o[q4] = v;
  }
}

// Any L * K: one 4-byte store per index.
template <int NMAX>
__global__ __launch_bounds__(kHashBlock) void hash_kernel_any(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    uint32_t* __restrict__ out) {
  const int64_t s = (int64_t)blockIdx.x * kHashBlock + threadIdx.x;
  if (s >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[NMAX];
  window<NMAX>(tokens + b * S, s, p.pad, tok);
  uint32_t* o = out + (b * S + s) * p.tables;
  for (int q = 0; q < p.tables; ++q) o[q] = table_index<NMAX>(tok, p.t[q]);
}

template <int LK, int NMAX>
hipError_t launch_vec(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                      dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((hash_kernel_vec<LK, NMAX>), grid, dim3(kHashBlock), 0, st, tokens, S,
                     p, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

template <int NMAX>
hipError_t launch(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                  dim3 grid, hipStream_t st) {
  switch (p.tables) {
    case 4: return launch_vec<4, NMAX>(tokens, S, p, out, grid, st);
    case 8: return launch_vec<8, NMAX>(tokens, S, p, out, grid, st);
    case 12: return launch_vec<12, NMAX>(tokens, S, p, out, grid, st);
    case 16: return launch_vec<16, NMAX>(tokens, S, p, out, grid, st);
    case 20: return launch_vec<20, NMAX>(tokens, S, p, out, grid, st);
    case 24: return launch_vec<24, NMAX>(tokens, S, p, out, grid, st);
    case 28: return launch_vec<28, NMAX>(tokens, S, p, out, grid, st);
    case 32: return launch_vec<32, NMAX>(tokens, S, p, out, grid, st);
    default:
      hipLaunchKernelGGL(hash_kernel_any<NMAX>, grid, dim3(kHashBlock), 0, st, tokens, S, p,
                         reinterpret_cast<uint32_t*>(out));
      return hipGetLastError();
  }
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
  int nmax = 1;
  for (int l = 0; l < L; ++l) {
    nmax = ngram[l] > nmax ? ngram[l] : nmax;
    for (int j = 0; j < K; ++j) {
      const int q = l * K + j;
      for (int i = 0; i < kMaxN; ++i)
        p.t[q].mult[i] = i < ngram[l] ? mult[(int64_t)q * kMaxN + i] : 0;
      p.t[q].mod = table_size[q];
      p.t[q].recip = UINT64_MAX / table_size[q];
    }
  }
  const dim3 grid((unsigned)((S + kHashBlock - 1) / kHashBlock), (unsigned)B);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (nmax) {
    case 1: e = launch<1>(tokens, S, p, out, grid, st); break;
    case 2: e = launch<2>(tokens, S, p, out, grid, st); break;
    case 3: e = launch<3>(tokens, S, p, out, grid, st); break;
    default: e = launch<4>(tokens, S, p, out, grid, st); break;
  }
  return e == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}
