// Hashed multi-table gather of the Engram memory (zhichai.net TileKernels
// page, section "5. Engram": N-gram hashed embedding tables with O(1)
// retrieval) for AMD MI355X (gfx950), and its C ABI entry point
// tk_engram_gather declared in include/tk_engram.h.
//
// The Q tables are packed in one bf16 buffer [total_rows, d]; table q holds
// rows [row_offset[q], row_offset[q] + rows[q]). For token t and table q,
//   out[t][q][:] = table_data[row_offset[q] + idx[t][q]][:]
// if 0 <= idx[t][q] < rows[q], else a zero row. Every index is checked
// against its table before the row is read, so no index, however bad,
// reads outside the buffer.
//
// One workgroup per token: its Q rows are Q * d / 8 16-byte chunks, written
// to a contiguous stretch of `out`; each thread moves up to four chunks at a
// time (all four loads issued before the stores). The token's Q indices are
// staged in LDS by one load, and each thread works out where its chunks live
// while that load is in flight, so the row loads issue right after one
// barrier instead of each waiting on a global index fetch of its own; that
// takes a memory round trip out of every chunk's dependency chain. Table
// reads are plain loads (common N-grams repeat, so rows can be re-used from
// cache); the output is streamed with nontemporal stores.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tk_engram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherBlock = 256;
static_assert(kGatherBlock >= TK_ENGRAM_GATHER_MAX_TABLES,
              "one thread per table stages the token's indices");
constexpr int kGatherUnroll = 4;

struct GatherParams {
  int64_t row_offset[TK_ENGRAM_GATHER_MAX_TABLES];
  uint32_t rows[TK_ENGRAM_GATHER_MAX_TABLES];
  int32_t tables;       // Q
  int32_t cpr;          // 16-byte chunks per row, d / 8
};

__global__ __launch_bounds__(kGatherBlock) void gather_kernel(
    const int32_t* __restrict__ idx, const u32x4* __restrict__ table,
    GatherParams p, u32x4* __restrict__ out) {
  __shared__ int32_t sidx[TK_ENGRAM_GATHER_MAX_TABLES];
  const int64_t t = blockIdx.x;
  const int n = p.tables * p.cpr;
  if (threadIdx.x < p.tables) sidx[threadIdx.x] = idx[t * p.tables + threadIdx.x];

  // Where this thread's next kGatherUnroll chunks come from: table q, the
  // chunk's offset within the packed buffer at row 0 of that table, and the
  // table's row count (0 for a chunk past the token's end, which then reads
  // nothing). The first group is located while the index load is in flight.
  int q[kGatherUnroll];
  int64_t base[kGatherUnroll];
  uint32_t lim[kGatherUnroll];
  auto locate = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int j = j0 + u * kGatherBlock;
      const int qq = j < n ? j / p.cpr : 0;
      q[u] = qq;
      base[u] = p.row_offset[qq] * p.cpr + (j - qq * p.cpr);
      lim[u] = j < n ? p.rows[qq] : 0u;
    }
  };
  locate(threadIdx.x);
  __syncthreads();

  u32x4* to = out + t * n;
  for (int j0 = threadIdx.x; j0 < n; j0 += kGatherUnroll * kGatherBlock) {
    u32x4 v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int32_t i = sidx[q[u]];
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (i >= 0 && (uint32_t)i < lim[u]) v[u] = table[base[u] + (int64_t)i * p.cpr];
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int j = j0 + u * kGatherBlock;
      if (j < n) __builtin_nontemporal_store(v[u], to + j);
    }
    if (j0 + kGatherUnroll * kGatherBlock < n) locate(j0 + kGatherUnroll * kGatherBlock);
  }
}

}  // namespace

extern "C" tk_status tk_engram_gather(const int32_t* idx, int64_t T, int32_t Q,
                                      const uint16_t* table_data, int64_t total_rows,
                                      int64_t d, const int64_t* row_offset,
                                      const uint32_t* rows, uint16_t* out,
                                      void* stream) {
  if (T < 0 || Q < 1 || d <= 0 || total_rows < 0) return TK_ERR_SHAPE;
  if (d % 8 != 0) return TK_ERR_ALIGN;
  if (Q > TK_ENGRAM_GATHER_MAX_TABLES || d > TK_ENGRAM_GATHER_MAX_D) return TK_ERR_UNSUPPORTED;
  if (!row_offset || !rows) return TK_ERR_NULL;
  for (int q = 0; q < Q; ++q)
    if (row_offset[q] < 0 || row_offset[q] > total_rows ||
        (int64_t)rows[q] > total_rows - row_offset[q])
      return TK_ERR_VALUE;
  if (T == 0) return TK_SUCCESS;
  if (!idx || !table_data || !out) return TK_ERR_NULL;
  if (((uintptr_t)idx & 3u) || ((uintptr_t)table_data & 15u) || ((uintptr_t)out & 15u))
    return TK_ERR_ALIGN;
  if (T > 0x7FFFFFFF) return TK_ERR_UNSUPPORTED;

  GatherParams p = {};
  p.tables = Q;
  p.cpr = (int32_t)(d / 8);
  for (int q = 0; q < Q; ++q) {
    p.row_offset[q] = row_offset[q];
    p.rows[q] = rows[q];
  }
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)T), dim3(kGatherBlock), 0,
                     reinterpret_cast<hipStream_t>(stream), idx,
                     reinterpret_cast<const u32x4*>(table_data), p,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError() == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}
