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
// quotient q = mulhi64(h, floor((2^64 - 1) / M)), which is at most 1 below
// floor(h / M), followed by one conditional subtraction in 32 bits.
//
// The kernel has no branches on N. Branching on a table's N made each wave
// wait for that table's parameters from the scalar cache before it could go
// on, which cost a third of the throughput. Instead, each table's number of
// products is fixed at compile time:
//   - two layers of eight tables (the layout the pages describe) have an
//     instance for every pair of orders (N0, N1), so a 2-gram table runs
//     two products and a 3-gram table three;
//   - every other layout runs NMAX products (the largest N of any layer) in
//     every table, with the multipliers of positions i >= N set to 0 on the
//     host: a product with 0 leaves the XOR unchanged, so the result is the
//     N-gram hash of the table's own layer.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tk_engram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTables = TK_ENGRAM_HASH_MAX_TABLES;  // L * K
constexpr int kMaxN = TK_ENGRAM_HASH_MAX_NGRAM;
constexpr int kHashBlock = 256;
constexpr int kWave = 64;
static_assert(kHashBlock % kWave == 0, "a block holds whole waves");

struct TableParams {
  uint64_t mult[kMaxN];  // multiplier of window position i; 0 for i >= N
  uint64_t recip;        // floor((2^64 - 1) / M)
  uint32_t mod;          // M
  uint32_t neg_r1m;      // -(floor(recip / 2^32) * M) mod 2^32
};

struct HashParams {
  TableParams t[kMaxTables];
  int32_t tables;  // L * K
  uint32_t pad;
};

// Layers of kPairK tables each, two of them: the layout with an instance per
// pair of N-gram orders.
constexpr int kPairK = 8;

// h mod m for 1 <= m <= 2^31, with R = floor((2^64 - 1) / m).
//
// The quotient q = floor(h R / 2^64) is at most one below floor(h / m):
// R > 2^64 / m - 1 when m is not a power of two (R = floor(2^64 / m) then),
// and R = 2^64 / m - 1 when it is, so in both cases
// h R / 2^64 > h / m - h / 2^64 > h / m - 1. Hence r = h - q m lies in
// [0, 2m), below 2^32, and one conditional subtraction finishes it.
//
// Since r < 2^32, only the low 32 bits of q and of q m matter. With
// h = h1 2^32 + h0 and R = R1 2^32 + R0,
//   q = h1 R1 + floor(A / 2^32),   A = h1 R0 + h0 R1 + floor(h0 R0 / 2^32),
// and the bits of A above 64 only reach bits of q above 31, so A is summed
// modulo 2^64. Then, modulo 2^32,
//   r = h0 - q m = h0 + h1 c - floor(A / 2^32) m,   c = -(R1 m),
// with c precomputed per table, so that h0 + h1 c is one 32 x 32 + 64-bit
// multiply-add on h itself. The subtraction uses min(r, r - m): below m,
// r - m wraps above r.
__device__ __forceinline__ uint32_t mod_exact(uint64_t h, uint64_t recip, uint32_t m,
                                              uint32_t neg_r1m) {
  const uint32_t h0 = (uint32_t)h, h1 = (uint32_t)(h >> 32);
  const uint32_t r0 = (uint32_t)recip, r1 = (uint32_t)(recip >> 32);
  const uint64_t a = (uint64_t)h0 * r1 + ((uint64_t)h1 * r0 + __umulhi(h0, r0));
  const uint32_t r = h0 + h1 * neg_r1m - (uint32_t)(a >> 32) * m;
  return min(r, r - m);
}

// The index of one table from its N products (N <= NMAX; the window holds
// NMAX tokens).
template <int NMAX, int N = NMAX>
__device__ __forceinline__ uint32_t table_index(const uint32_t (&tok)[NMAX],
                                                const TableParams& t) {
  static_assert(N >= 1 && N <= NMAX, "a table uses at most the window's tokens");
  // tok * mult mod 2^64 = tok * lo(mult) + (tok * hi(mult) mod 2^32) 2^32:
  // written so, each product is one 32-bit multiply and one multiply-add
  uint64_t h = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t m0 = (uint32_t)t.mult[i], m1 = (uint32_t)(t.mult[i] >> 32);
    h ^= (uint64_t)tok[i] * m0 + ((uint64_t)(tok[i] * m1) << 32);
  }
  return mod_exact(h, t.recip, t.mod, t.neg_r1m);
}

// tok[i] = token at position s - i of the sequence, `pad` before its start
// (and for positions s >= S, whose indices are never stored).
template <int NMAX>
__device__ __forceinline__ void window(const int32_t* __restrict__ seq, int64_t s, int64_t S,
                                       uint32_t pad, uint32_t (&tok)[NMAX]) {
#pragma unroll
  for (int i = 0; i < NMAX; ++i) tok[i] = (s < S && s - i >= 0) ? (uint32_t)seq[s - i] : pad;
}

// The 64 tokens of a wave own one contiguous stretch of the output, 64 * LK
// indices. Each lane hashes its token into the wave's slice of LDS, and the
// wave then writes the stretch with consecutive lanes on consecutive
// 16-byte (or 4-byte) words, so every store instruction covers one
// contiguous span. Written straight from the registers, lane l's indices
// would sit LK * 4 bytes apart, and each store instruction would touch 64
// separate pieces of cache lines: that form took 1.6 times as long.
// Only the wave's own lanes touch its slice, so a wave-level fence orders
// the LDS writes before the reads. The stores carry the nontemporal hint:
// with it the 4.2 M-token hash took 49 us instead of 59 us, although a plain
// write stream of the same size is faster with cached stores (39 us against
// 45 us).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// L * K == LK, a multiple of 4: the output leaves in 16-byte stores. Tables
// q < LK / 2 run N0 products and the others N1 (both NMAX unless the layout
// is two layers of kPairK tables).
template <int LK, int NMAX, int N0 = NMAX, int N1 = NMAX>
__global__ __launch_bounds__(kHashBlock) void hash_kernel_vec(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    u32x4* __restrict__ out) {
  constexpr int Q4 = LK / 4;  // 16-byte words per token
  __shared__ u32x4 stage[kHashBlock * Q4];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t s0 = (int64_t)blockIdx.x * kHashBlock + wave * kWave;  // wave's first token
  if (s0 >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[NMAX];
  window<NMAX>(tokens + b * S, s0 + lane, S, p.pad, tok);
  u32x4* ws = stage + wave * kWave * Q4;
#pragma unroll
  for (int q4 = 0; q4 < Q4; ++q4) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = 4 * q4 + e;
      v[e] = q < LK / 2 ? table_index<NMAX, N0>(tok, p.t[q]) : table_index<NMAX, N1>(tok, p.t[q]);
    }
    ws[lane * Q4 + q4] = v;
  }
  wave_lds_sync();
  const int64_t ntok = S - s0 < kWave ? S - s0 : kWave;  // tokens of this wave
  u32x4* o = out + (b * S + s0) * Q4;
#pragma unroll
  for (int j = 0; j < Q4; ++j) {
    const int c = j * kWave + lane;
    if (c < ntok * Q4) __builtin_nontemporal_store(ws[c], o + c);
  }
}

// Any L * K (at most kMaxTables): the output leaves in 4-byte stores.
template <int NMAX>
__global__ __launch_bounds__(kHashBlock) void hash_kernel_any(
    const int32_t* __restrict__ tokens, int64_t S, HashParams p,
    uint32_t* __restrict__ out) {
  __shared__ uint32_t stage[kHashBlock * kMaxTables];
  const int LK = p.tables;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t s0 = (int64_t)blockIdx.x * kHashBlock + wave * kWave;
  if (s0 >= S) return;
  const int64_t b = blockIdx.y;
  uint32_t tok[NMAX];
  window<NMAX>(tokens + b * S, s0 + lane, S, p.pad, tok);
  uint32_t* ws = stage + wave * kWave * kMaxTables;
  for (int q = 0; q < LK; ++q) ws[lane * LK + q] = table_index<NMAX>(tok, p.t[q]);
  wave_lds_sync();
  const int64_t ntok = S - s0 < kWave ? S - s0 : kWave;
  uint32_t* o = out + (b * S + s0) * LK;
  for (int c = lane; c < ntok * LK; c += kWave) __builtin_nontemporal_store(ws[c], o + c);
}

template <int LK, int NMAX, int N0 = NMAX, int N1 = NMAX>
hipError_t launch_vec(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                      dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((hash_kernel_vec<LK, NMAX, N0, N1>), grid, dim3(kHashBlock), 0, st, tokens,
                     S, p, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

// Two layers of kPairK tables whose orders differ: the instance for the pair
// (n0, n1), max(n0, n1) == NMAX.
template <int NMAX>
hipError_t launch_pair(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                       dim3 grid, hipStream_t st, int n0, int n1) {
  constexpr int LK = 2 * kPairK;
  const int lo = n0 < n1 ? n0 : n1;
  const bool up = n0 < n1;  // the first layer has the lower order
  switch (lo) {
    case 1:
      return up ? launch_vec<LK, NMAX, 1, NMAX>(tokens, S, p, out, grid, st)
                : launch_vec<LK, NMAX, NMAX, 1>(tokens, S, p, out, grid, st);
    case 2:
      if constexpr (NMAX > 2)
        return up ? launch_vec<LK, NMAX, 2, NMAX>(tokens, S, p, out, grid, st)
                  : launch_vec<LK, NMAX, NMAX, 2>(tokens, S, p, out, grid, st);
      break;
    case 3:
      if constexpr (NMAX > 3)
        return up ? launch_vec<LK, NMAX, 3, NMAX>(tokens, S, p, out, grid, st)
                  : launch_vec<LK, NMAX, NMAX, 3>(tokens, S, p, out, grid, st);
      break;
    default:
      break;
  }
  return launch_vec<LK, NMAX>(tokens, S, p, out, grid, st);
}

// n0, n1: the orders of the two layers when the layout is two layers of
// kPairK tables, else 0.
template <int NMAX>
hipError_t launch(const int32_t* tokens, int64_t S, const HashParams& p, void* out,
                  dim3 grid, hipStream_t st, int n0, int n1) {
  if (n0 > 0 && n0 != n1) return launch_pair<NMAX>(tokens, S, p, out, grid, st, n0, n1);
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
      p.t[q].neg_r1m = 0u - (uint32_t)(p.t[q].recip >> 32) * table_size[q];
    }
  }
  const bool pair = L == 2 && K == kPairK;
  const int n0 = pair ? ngram[0] : 0, n1 = pair ? ngram[1] : 0;
  const dim3 grid((unsigned)((S + kHashBlock - 1) / kHashBlock), (unsigned)B);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (nmax) {
    case 1: e = launch<1>(tokens, S, p, out, grid, st, n0, n1); break;
    case 2: e = launch<2>(tokens, S, p, out, grid, st, n0, n1); break;
    case 3: e = launch<3>(tokens, S, p, out, grid, st, n0, n1); break;
    default: e = launch<4>(tokens, S, p, out, grid, st, n0, n1); break;
  }
  return e == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}
