// Engram gate for AMD MI355X (gfx950): HIP kernels and the C ABI of
// include/tk_engram.h.
//
// The operation is the gate of the zhichai.net TileKernels page, section
// "5. Engram" (gate formula), with its backward and the weight-gradient
// reduction that the same section lists as separate kernels.
//
// Everything on this path streams bf16 rows from HBM and reduces each row to
// a handful of scalars; nothing is a dense contraction, so no matrix cores
// are used. Each kernel is built around one idea: about one workgroup of W
// waves per CU walks the rows b, b + G, b + 2G, ... (G workgroups, b its
// logical number) one row at a time, so the rows in flight across the chip
// stay in one sliding window of the tensors; the row is split across the
// W*64 threads in 16-byte chunks (8 bf16), thread `tid` owning chunks tid,
// tid + W*64, ... so that every load and store instruction of a wave covers
// 1 KiB of contiguous memory. While a row is reduced and written, the loads
// of the next rows are already in flight.
//
// Algebra used by both passes. With w_i = wh_i * we_i (the product of the
// two RMSNorm weights) and the normalised rows x^ = r_x x, k^ = r_k k,
//   d = r_x r_k sum_i x_i k_i w_i,
// and the chain rule through out = x + gate * v gives per row
//   dd = (sum_i gout_i v_i) * g (1 - g) / (2 sqrt(max(|z|, clamp))) / sqrt(H)
//   dx_i = gout_i + (dd r_x) w_i k^_i - (dd r_x d / H) x^_i,
//   dk_i =          (dd r_k) w_i x^_i - (dd r_k d / H) k^_i,
//   dv_i = g gout_i,
// and the weight gradients share one column vector c_i = sum_t dd_t x^_ti k^_ti:
//   dL/dwh_i = we_i c_i,   dL/dwe_i = wh_i c_i.
//
// Precision and range: every row sum (of x^2, k^2, x k w and gout v) is
// accumulated in fp64 from exact fp64 products of the bf16 values, and the
// row scalars r_x, r_k, d and dd are fp64. The dot product that decides the
// gate near z = 0 thus carries only relative rounding error, and no finite
// bf16 row overflows or underflows on its way to the gate: the elementwise
// work is fp32 on the normalised rows, whose mean squares are at most 1,
// with coefficients rounded to fp32 only after they are formed in fp64.
// The gate itself uses the hardware's fp32 square root, exp2 and reciprocal
// (about 1 ulp each), which move it by < 1e-7. The backward takes the
// sigmoid's derivative g (1 - g) with 1 - g evaluated as sigmoid(-s), so it
// keeps its relative precision where the gate saturates toward 1.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <algorithm>
#include <cstdint>
#include <mutex>

#include "tk_engram.h"

// Device memory of tk_engram_gate_bwd_reduce_noalloc (see scratch_of below).
static __device__ __align__(256) float scratch[TK_ENGRAM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- bf16 packing --------------------------------------------------------

__device__ __forceinline__ void unpack8(const u32x4 u, float f[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(u[q] << 16);
    f[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
  }
}

// Round to nearest even; gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  u32x4 u;
#pragma unroll
  for (int q = 0; q < 4; ++q) u[q] = pack2(f[2 * q], f[2 * q + 1]);
  return u;
}

// ---- wave reductions ---------------------------------------------------------

// Sum over the 64 lanes of a wave, returned to every lane with the same bits.
// Within each row of 16 lanes, four DPP steps combine lanes i^1, i^2 (quad
// permutes), 7-i (half-row mirror) and 15-i (row mirror); IEEE addition is
// commutative, so after each step all lanes of the group hold identical
// values. The four row sums are then read from lanes 0, 16, 32 and 48 and
// added in a fixed order. Everything stays in VALU/SALU, with none of the
// LDS round trips of a permute-based butterfly.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp_step(float v) {
  return v + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_step(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = dpp_u32<CTRL>((uint32_t)u);
  const uint64_t hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return v + __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ double lane_value(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, lo | (hi << 32));
}

template <class F>
__device__ __forceinline__ F wave_sum(F v) {
  v = dpp_step<kDppXor1>(v);
  v = dpp_step<kDppXor2>(v);
  v = dpp_step<kDppHalfMirror>(v);
  v = dpp_step<kDppMirror>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// ---- per-thread slice of a row ---------------------------------------------

// Chunk j of thread `tid` is 16-byte chunk j * NT + tid of the row. Every row
// is read and written exactly once, so loads and stores carry the
// nontemporal hint (streamed, not kept in the caches).
template <int NT, int C, bool FULL>
__device__ __forceinline__ void load_row(const u32x4* __restrict__ row, int tid,
                                         int nchunk, u32x4 (&dst)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if (FULL || c < nchunk) {
      dst[j] = __builtin_nontemporal_load(row + c);
    } else {
      dst[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_chunk(u32x4* __restrict__ p, const u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

// The RMSNorm weights as the gate kernels receive them: wh and we (fp32
// [H]), or their product w = wh * we in fp64 (the fused weight of the
// "5. Engram" section's weight preprocessing), read as it is (FUSED).
struct WeightsIn {
  const f32x4* wh;
  const f32x4* we;
  const f64x2* w;
};

// w_i = wh_i * we_i for the thread's columns, exactly (the product of two
// fp32 values is exact in fp64), or the fused weight as given. The
// elementwise backward uses its fp32 rounding, (float)w, which for a product
// of two fp32 values is the correctly rounded fp32 product.
template <int NT, int C, bool FULL, bool FUSED>
__device__ __forceinline__ void load_weights(const WeightsIn& in, int tid, int nchunk,
                                             double (&w64)[C][8]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if constexpr (FUSED) {
      f64x2 q[4] = {{0.0, 0.0}, {0.0, 0.0}, {0.0, 0.0}, {0.0, 0.0}};
      if (FULL || c < nchunk) {
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = in.w[4 * c + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w64[j][2 * u] = q[u][0];
        w64[j][2 * u + 1] = q[u][1];
      }
    } else {
      f32x4 a0 = {0, 0, 0, 0}, a1 = a0, b0 = a0, b1 = a0;
      if (FULL || c < nchunk) {
        a0 = in.wh[2 * c];
        a1 = in.wh[2 * c + 1];
        b0 = in.we[2 * c];
        b1 = in.we[2 * c + 1];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w64[j][e] = (double)a0[e] * (double)b0[e];
        w64[j][e + 4] = (double)a1[e] * (double)b1[e];
      }
    }
  }
}

// Where a thread keeps w_i = wh_i * we_i (fp64) for its columns: in
// registers, or in LDS as thread-private storage (each thread reads back
// only what it wrote itself, so no barrier is needed), which frees 16 * C
// VGPRs for deeper row prefetch. Element e of the thread's chunk j lives at
// wl[e * NT * C + j * NT + tid], so a wave's reads are 64 consecutive
// doubles.
template <int C>
struct WeightsReg {
  double w[C][8];
  __device__ __forceinline__ double get(int j, int e) const { return w[j][e]; }
};

template <int NT, int C>
struct WeightsLds {
  double* wl;
  int tid;
  __device__ __forceinline__ double get(int j, int e) const {
    return wl[e * NT * C + j * NT + tid];
  }
};

template <int NT, int C>
__device__ __forceinline__ WeightsLds<NT, C> stage_weights(const double (&w64)[C][8],
                                                           double* wl, int tid) {
#pragma unroll
  for (int j = 0; j < C; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) wl[e * NT * C + j * NT + tid] = w64[j][e];
  return WeightsLds<NT, C>{wl, tid};
}

struct RowScalars {
  double r_x, r_k, d;  // 1/sqrt(mean(x^2) + eps), likewise for k, the dot d
  float z, g, gm;      // z = d / sqrt(H), gate, 1 - gate
};

// 1/sqrt(m) for m >= eps: the hardware estimate and one Newton step.
__device__ __forceinline__ double rsqrt64(double m) {
  const double r = __builtin_amdgcn_rsq(m);
  return r * fma(-0.5 * m * r, r, 1.5);
}

// Gate of one row from its three sums (formula of the section "5. Engram").
// Everything that scales with the data stays in fp64, so no row of finite
// bf16 values overflows or underflows on its way to z, which is O(H^(1/2)).
__device__ __forceinline__ RowScalars row_gate(double sum_xx, double sum_kk,
                                               double sum_xkw, double eps,
                                               double inv_h, double inv_sqrt_h) {
  RowScalars s;
  s.r_x = rsqrt64(fma(sum_xx, inv_h, eps));
  s.r_k = rsqrt64(fma(sum_kk, inv_h, eps));
  s.d = sum_xkw * s.r_x * s.r_k;
  s.z = (float)(s.d * inv_sqrt_h);
  // signed_sqrt: sign(z) sqrt|z|, with sign(0) = 0
  const float sq = copysignf(__builtin_amdgcn_sqrtf(fabsf(s.z)), s.z);
  // sigmoid(sq) = 1 / (1 + 2^(-sq log2 e))
  const float e = __builtin_amdgcn_exp2f(-sq * 1.4426950408889634f);
  s.g = __builtin_amdgcn_rcpf(1.0f + e);
  // 1 - gate = sigmoid(-sq), evaluated as such: 1 - g would keep only g's
  // rounding error once the gate is within a few ulp of 1 (sq beyond about
  // 10) and be 0 beyond about 17. Only the backward uses it.
  s.gm = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sq * 1.4426950408889634f));
  return s;
}

// Row pipelining. A workgroup keeps D row buffers in registers: while one
// row is reduced and written, the loads of the next D - 1 rows it owns are in
// flight. The buffers rotate by unrolling the row loop D times (no register
// copies, which would make the compiler wait for the prefetch), and every
// prefetch is issued unconditionally with its row index clamped to the
// block's last row of the launch, so the final redundant loads re-read that
// row (a branch around them measured slower).
//
// Cross-wave sums go through LDS slots indexed by row parity: a slot is
// rewritten two rows later, after every thread has passed the barrier of
// the row in between, so one barrier per row suffices.

// Which rows a workgroup walks. With G workgroups, block b owns rows
// b, b + G, b + 2G, ... (row t belongs to block t mod G), which keeps the rows
// in flight across the chip inside one sliding window of the tensors. A
// launch covers iterations [iter0, iter0 + iters) of that walk: block b takes
// rows b + (iter0 + i) G, i = 0 .. rows_of(first_row(b)) - 1, never beyond T.
// A long walk is split into several such launches (epochs): on MI355X a
// launch of many rows per block loses bandwidth as it goes, most plausibly
// because the blocks drift apart and widen the window of rows in flight, and
// each launch boundary brings them back in step.
struct RowWalk {
  int64_t T;
  int64_t row_step;  // G
  int64_t iter0;
  int64_t iters;
  __device__ __forceinline__ int64_t first_row(int64_t blk) const {
    return blk + iter0 * row_step;
  }
  __device__ __forceinline__ int64_t rows_of(int64_t first) const {
    if (first >= T) return 0;
    const int64_t n = (T - first + row_step - 1) / row_step;
    return n < iters ? n : iters;
  }
};

// The workgroup's logical number b in the walk above. The dispatcher hands
// workgroups to the 8 XCDs in turn (hardware workgroup w runs on XCD w mod 8),
// so numbering them XCD by XCD gives each XCD a contiguous slab of the rows
// in flight instead of every 8th row; the backward at H = 7168 gains about
// 1%. It is a fixed permutation of the grid, so which rows and which partial
// slot belong to logical block b, and hence every result bit, are unchanged.
// Grids that 8 does not divide keep the plain numbering.
__device__ __forceinline__ int64_t xcd_slab_block() {
  const int64_t w = blockIdx.x, G = gridDim.x;
  return (G & 7) ? w : (w & 7) * (G >> 3) + (w >> 3);
}

// ---- forward ---------------------------------------------------------------

template <int C>
struct FwdBuf {
  u32x4 x[C], k[C], v[C];
};

template <int NT, int C, bool FULL>
__device__ __forceinline__ void fwd_load(FwdBuf<C>& b, const u32x4* __restrict__ x,
                                         const u32x4* __restrict__ k,
                                         const u32x4* __restrict__ v, int64_t row,
                                         int nchunk, int tid) {
  const int64_t o = row * nchunk;
  load_row<NT, C, FULL>(x + o, tid, nchunk, b.x);
  load_row<NT, C, FULL>(k + o, tid, nchunk, b.k);
  load_row<NT, C, FULL>(v + o, tid, nchunk, b.v);
}

template <int W, int C, bool FULL, class WT>
__device__ __forceinline__ void fwd_row(const FwdBuf<C>& b, int64_t r, int slot,
                                        int tid, int nchunk, const WT& w64,
                                        double (&red)[2][3][W],
                                        u32x4* __restrict__ out,
                                        float* __restrict__ gate, double eps,
                                        double inv_h, double inv_sqrt_h) {
  constexpr int NT = W * kWave;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  double sxx = 0.0, skk = 0.0, sxkw = 0.0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    float xf[8], kf[8];
    unpack8(b.x[j], xf);
    unpack8(b.k[j], kf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // squares and x_i k_i are exact in fp64 (8-bit significands) at any
      // bf16 magnitude
      const double xd = xf[e], kd = kf[e];
      sxx = fma(xd, xd, sxx);
      skk = fma(kd, kd, skk);
      sxkw = fma(xd * kd, w64.get(j, e), sxkw);
    }
  }
  sxx = wave_sum(sxx);
  skk = wave_sum(skk);
  sxkw = wave_sum(sxkw);
  if (lane == 0) {
    red[slot][0][wave] = sxx;
    red[slot][1][wave] = skk;
    red[slot][2][wave] = sxkw;
  }
  __syncthreads();
  double txx = 0.0, tkk = 0.0, txkw = 0.0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    txx += red[slot][0][i];
    tkk += red[slot][1][i];
    txkw += red[slot][2][i];
  }
  const RowScalars s = row_gate(txx, tkk, txkw, eps, inv_h, inv_sqrt_h);

  const int64_t o = r * nchunk;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if (FULL || c < nchunk) {
      float xf[8], vf[8], of[8];
      unpack8(b.x[j], xf);
      unpack8(b.v[j], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) of[e] = fmaf(s.g, vf[e], xf[e]);
      store_chunk(out + o + c, pack8(of));
    }
  }
  if (tid == 0) gate[r] = s.g;
}

template <int W, int C, bool FULL, int D, bool FUSED>
__global__ __launch_bounds__(W * kWave) void gate_fwd_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ k,
    const u32x4* __restrict__ v, WeightsIn wts, u32x4* __restrict__ out,
    float* __restrict__ gate, RowWalk walk, int nchunk, double eps, double inv_h,
    double inv_sqrt_h) {
  constexpr int NT = W * kWave;
  const int tid = threadIdx.x;
  __shared__ double red[2][3][W];

  const int64_t blk = xcd_slab_block();
  const int64_t first = walk.first_row(blk);
  const int64_t n = walk.rows_of(first);
  if (n <= 0) return;
  const int64_t step = walk.row_step;
  auto row = [&](int64_t i) { return first + (i < n ? i : n - 1) * step; };

  // The weights are loaded before the first rows: loads complete in order,
  // so the first row's dot product then waits for them alone.
  WeightsReg<C> w64;
  load_weights<NT, C, FULL, FUSED>(wts, tid, nchunk, w64.w);
  FwdBuf<C> buf[D];
#pragma unroll
  for (int s = 0; s + 1 < D; ++s) fwd_load<NT, C, FULL>(buf[s], x, k, v, row(s), nchunk, tid);

  for (int64_t i = 0;; i += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      fwd_load<NT, C, FULL>(buf[(s + D - 1) % D], x, k, v, row(i + s + D - 1), nchunk,
                            tid);
      fwd_row<W, C, FULL>(buf[s], row(i + s), (int)((i + s) & 1), tid, nchunk, w64,
                          red, out, gate, eps, inv_h, inv_sqrt_h);
      if (i + s + 1 >= n) return;
    }
  }
}

// ---- backward --------------------------------------------------------------

template <int C>
struct BwdBuf {
  u32x4 g[C], x[C], k[C], v[C];
};

template <int NT, int C, bool FULL>
__device__ __forceinline__ void bwd_load(BwdBuf<C>& b, const u32x4* __restrict__ gout,
                                         const u32x4* __restrict__ x,
                                         const u32x4* __restrict__ k,
                                         const u32x4* __restrict__ v, int64_t row,
                                         int nchunk, int tid) {
  const int64_t o = row * nchunk;
  load_row<NT, C, FULL>(gout + o, tid, nchunk, b.g);
  load_row<NT, C, FULL>(v + o, tid, nchunk, b.v);
  load_row<NT, C, FULL>(x + o, tid, nchunk, b.x);
  load_row<NT, C, FULL>(k + o, tid, nchunk, b.k);
}

template <int W, int C, bool FULL, class WT, class AFTER>
__device__ __forceinline__ void bwd_row(const BwdBuf<C>& b, int64_t r, int slot,
                                        const AFTER& after, int tid, int nchunk,
                                        const WT& w64,
                                        float (&cacc)[C][8],
                                        double (&red)[2][4][W],
                                        u32x4* __restrict__ dx,
                                        u32x4* __restrict__ dk,
                                        u32x4* __restrict__ dv, double eps,
                                        float clamp, double inv_h,
                                        double inv_sqrt_h) {
  constexpr int NT = W * kWave;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // the forward's sums in the forward's order, so the gate has its bits
  double sxx = 0.0, skk = 0.0, sxkw = 0.0, sgv = 0.0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    float gf[8], xf[8], kf[8], vf[8];
    unpack8(b.g[j], gf);
    unpack8(b.v[j], vf);
    unpack8(b.x[j], xf);
    unpack8(b.k[j], kf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xd = xf[e], kd = kf[e];
      sgv = fma((double)gf[e], (double)vf[e], sgv);
      sxx = fma(xd, xd, sxx);
      skk = fma(kd, kd, skk);
      sxkw = fma(xd * kd, w64.get(j, e), sxkw);
    }
  }
  sxx = wave_sum(sxx);
  skk = wave_sum(skk);
  sgv = wave_sum(sgv);
  sxkw = wave_sum(sxkw);
  if (lane == 0) {
    red[slot][0][wave] = sxx;
    red[slot][1][wave] = skk;
    red[slot][2][wave] = sxkw;
    red[slot][3][wave] = sgv;
  }
  __syncthreads();
  double txx = 0.0, tkk = 0.0, txkw = 0.0, tgv = 0.0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    txx += red[slot][0][i];
    tkk += red[slot][1][i];
    txkw += red[slot][2][i];
    tgv += red[slot][3][i];
  }
  const RowScalars s = row_gate(txx, tkk, txkw, eps, inv_h, inv_sqrt_h);
  // gate = sigmoid(sq): d gate / d sq = g (1 - g) = g gm;
  // sq = signed_sqrt(z): d sq / dz = 1 / (2 sqrt(max(|z|, clamp)));
  // z = d / sqrt(H).
  const float half_dsq = 0.5f * __builtin_amdgcn_rsqf(fmaxf(fabsf(s.z), clamp));
  const double dd = tgv * (double)(s.g * s.gm) * (double)half_dsq * inv_sqrt_h;
  // With x^ = r_x x and k^ = r_k k, whose mean squares are at most 1:
  //   dx = gout + (dd r_x) w k^ - (dd r_x d / H) x^
  //   dk =        (dd r_k) w x^ - (dd r_k d / H) k^
  //   c += dd x^ k^
  // Every coefficient is formed in fp64 before it is rounded to fp32.
  const float rxf = (float)s.r_x, rkf = (float)s.r_k;
  const float ax = (float)(dd * s.r_x), bx = (float)(dd * s.r_x * s.d * inv_h);
  const float ak = (float)(dd * s.r_k), bk = (float)(dd * s.r_k * s.d * inv_h);
  const float cd = (float)dd;

  const int64_t o = r * nchunk;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if (FULL || c < nchunk) {
      float gf[8], xf[8], kf[8], ox[8], ok[8], ov[8];
      unpack8(b.g[j], gf);
      unpack8(b.x[j], xf);
      unpack8(b.k[j], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = (float)w64.get(j, e);
        const float xh = rxf * xf[e], kh = rkf * kf[e];
        ox[e] = fmaf(-bx, xh, fmaf(ax, w * kh, gf[e]));
        ok[e] = fmaf(-bk, kh, ak * (w * xh));
        ov[e] = s.g * gf[e];
        cacc[j][e] = fmaf(cd, xh * kh, cacc[j][e]);
      }
      store_chunk(dx + o + c, pack8(ox));
      store_chunk(dk + o + c, pack8(ok));
      store_chunk(dv + o + c, pack8(ov));
    }
  }
  after();
}

template <int W, int C, bool FULL, int D, bool WLDS, bool FUSED>
__global__ __launch_bounds__(W * kWave) void gate_bwd_kernel(
    const u32x4* __restrict__ gout, const u32x4* __restrict__ x,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, WeightsIn wts,
    u32x4* __restrict__ dx, u32x4* __restrict__ dk, u32x4* __restrict__ dv,
    f32x4* __restrict__ partial, RowWalk walk, int nchunk, double eps,
    float clamp, double inv_h, double inv_sqrt_h, int carry) {
  constexpr int NT = W * kWave;
  const int tid = threadIdx.x;
  __shared__ double red[2][4][W];

  const int64_t blk = xcd_slab_block();
  f32x4* prow = partial + blk * (2 * nchunk);

  // c_i over this block's rows, for the thread's columns: from zero in the
  // first epoch, else from the previous epoch's partial row, so the sum runs
  // in the same order, with the same fp32 state, as one long walk.
  float cacc[C][8];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
    if (carry && (FULL || c < nchunk)) {
      lo = prow[2 * c];
      hi = prow[2 * c + 1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cacc[j][e] = lo[e];
      cacc[j][e + 4] = hi[e];
    }
  }

  const int64_t first = walk.first_row(blk);
  const int64_t n = walk.rows_of(first);

  if (n > 0) {
    const int64_t step = walk.row_step;
    auto row = [&](int64_t i) { return first + (i < n ? i : n - 1) * step; };
    // weights before the first rows (loads complete in order)
    double w64[C][8];
    load_weights<NT, C, FULL, FUSED>(wts, tid, nchunk, w64);
    BwdBuf<C> buf[D];
#pragma unroll
    for (int s = 0; s + 1 < D; ++s)
      bwd_load<NT, C, FULL>(buf[s], gout, x, k, v, row(s), nchunk, tid);
    auto walk_rows = [&](const auto& wts) {
      for (int64_t i = 0;; i += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
          BwdBuf<C>& nb = buf[(s + D - 1) % D];
          const int64_t next = row(i + s + D - 1);
          if constexpr (D >= 3) {
            // With two rows of loads in flight the prefetch is split: x and k
            // of the next row at the start of the iteration, grad_out and v
            // after this row's stores. Streams at equal offsets modulo 2 MiB
            // (separate allocations) then meet the same HBM banks less often;
            // about 1% faster at H = 7168, every bit the same. The plans with
            // three rows in flight are the wide ones (5, 6 or 7 waves of two
            // chunks per row); the two-wave plans run faster with two.
            const int64_t o = next * nchunk;
            load_row<NT, C, FULL>(x + o, tid, nchunk, nb.x);
            load_row<NT, C, FULL>(k + o, tid, nchunk, nb.k);
            __builtin_amdgcn_sched_barrier(0);
            auto after = [&]() {
              __builtin_amdgcn_sched_barrier(0);
              load_row<NT, C, FULL>(gout + o, tid, nchunk, nb.g);
              load_row<NT, C, FULL>(v + o, tid, nchunk, nb.v);
              __builtin_amdgcn_sched_barrier(0);
            };
            bwd_row<W, C, FULL>(buf[s], row(i + s), (int)((i + s) & 1), after, tid, nchunk,
                                wts, cacc, red, dx, dk, dv, eps, clamp, inv_h, inv_sqrt_h);
          } else {
            bwd_load<NT, C, FULL>(nb, gout, x, k, v, next, nchunk, tid);
            bwd_row<W, C, FULL>(buf[s], row(i + s), (int)((i + s) & 1), [] {}, tid, nchunk,
                                wts, cacc, red, dx, dk, dv, eps, clamp, inv_h, inv_sqrt_h);
          }
          if (i + s + 1 >= n) return;
        }
      }
    };
    if constexpr (WLDS) {
      __shared__ double wl[8 * NT * C];
      walk_rows(stage_weights<NT, C>(w64, wl, tid));
    } else {
      WeightsReg<C> wr;
#pragma unroll
      for (int j = 0; j < C; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) wr.w[j][e] = w64[j][e];
      walk_rows(wr);
    }
  }

  // This block's partial row of c.
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if (FULL || c < nchunk) {
      prow[2 * c] = f32x4{cacc[j][0], cacc[j][1], cacc[j][2], cacc[j][3]};
      prow[2 * c + 1] = f32x4{cacc[j][4], cacc[j][5], cacc[j][6], cacc[j][7]};
    }
  }
}

// ---- weight-gradient reduction -------------------------------------------

// 256 threads: kRedCols4 groups of 4 columns x kRedSlices strided slices of
// the partials. Each thread sums its slice (partials p = slice, slice + S,
// ...) in increasing p, with the loads of kRedUnroll partials in flight at a
// time; the slice sums are then added in increasing slice order. The order
// depends only on (P, H).
constexpr int kRedCols4 = 8;
constexpr int kRedSlices = 32;
constexpr int kRedUnroll = 8;

__global__ __launch_bounds__(kRedCols4* kRedSlices) void grad_w_reduce_kernel(
    const f32x4* __restrict__ partial, int64_t P, int nq,
    const f32x4* __restrict__ wh, const f32x4* __restrict__ we,
    f32x4* __restrict__ dwh, f32x4* __restrict__ dwe) {
  __shared__ f32x4 part[kRedSlices][kRedCols4];
  const int cx = threadIdx.x % kRedCols4;
  const int py = threadIdx.x / kRedCols4;
  const int q = blockIdx.x * kRedCols4 + cx;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (q < nq) {
    int64_t p = py;
    for (; p + (kRedUnroll - 1) * kRedSlices < P; p += kRedUnroll * kRedSlices) {
      f32x4 t[kRedUnroll];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) t[u] = partial[(p + u * kRedSlices) * nq + q];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) s += t[u];
    }
    for (; p < P; p += kRedSlices) s += partial[p * nq + q];
  }
  part[py][cx] = s;
  __syncthreads();
  if (py == 0 && q < nq) {
    f32x4 t = part[0][cx];
#pragma unroll
    for (int i = 1; i < kRedSlices; ++i) t += part[i][cx];
    dwh[q] = t * we[q];
    dwe[q] = t * wh[q];
  }
}

// ---- fused weight ------------------------------------------------------------

// w_i = wh_i * we_i in fp64: the product of two fp32 values is exact there.
__global__ __launch_bounds__(256) void fused_weight_kernel(const float* __restrict__ wh,
                                                           const float* __restrict__ we,
                                                           double* __restrict__ w, int64_t H) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < H) w[i] = (double)wh[i] * (double)we[i];
}

// ---- copy probe ------------------------------------------------------------

// Each block copies contiguous 16 KiB tiles (256 threads x 4 chunks), tiles
// dealt round-robin over the blocks; the remainder below one tile is copied
// chunk by chunk. Nontemporal like the gate kernels.
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void copy_probe_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  constexpr int64_t tile = 256 * kCopyUnroll;
  const int64_t ntile = n / tile;
  for (int64_t t = blockIdx.x; t < ntile; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
    u32x4 a[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      a[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) store_chunk(dst + base + u * 256, a[u]);
  }
  for (int64_t i = ntile * tile + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// ---- stream-mix probe -------------------------------------------------------

// R input streams and S output streams of n 16-byte chunks each, in the same
// tiled nontemporal pattern as the copy probe: output o is the XOR of all
// inputs plus o, so no load is dead. Measures the practical HBM ceiling of a
// kernel's read/write mix (the forward reads 3 and writes 1 stream, the
// backward reads 4 and writes 3).
struct StreamSet {
  const u32x4* in[TK_ENGRAM_PROBE_MAX_STREAMS];
  u32x4* out[TK_ENGRAM_PROBE_MAX_STREAMS];
};

template <int R, int S>
__global__ __launch_bounds__(256) void stream_probe_kernel(StreamSet st, int64_t n) {
  constexpr int64_t tile = 256 * kCopyUnroll;
  const int64_t ntile = n / tile;
  for (int64_t t = blockIdx.x; t < ntile; t += gridDim.x) {
    const int64_t base = t * tile + threadIdx.x;
    u32x4 a[R][kCopyUnroll];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        a[i][u] = __builtin_nontemporal_load(st.in[i] + base + u * 256);
#pragma unroll
    for (int o = 0; o < S; ++o)
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        u32x4 x = a[0][u];
#pragma unroll
        for (int i = 1; i < R; ++i) x ^= a[i][u] + (uint32_t)o;
        store_chunk(st.out[o] + base + u * 256, x);
      }
  }
  for (int64_t i = ntile * tile + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
#pragma unroll
    for (int o = 0; o < S; ++o) {
      u32x4 x = st.in[0][i];
#pragma unroll
      for (int k = 1; k < R; ++k) x ^= st.in[k][i] + (uint32_t)o;
      st.out[o][i] = x;
    }
  }
}

// ---- host side -------------------------------------------------------------

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

tk_status check_shape(int64_t T, int64_t H) {
  if (T < 0 || H <= 0) return TK_ERR_SHAPE;
  if (H % 8 != 0) return TK_ERR_ALIGN;
  if (H > TK_ENGRAM_MAX_H) return TK_ERR_UNSUPPORTED;
  return TK_SUCCESS;
}

// RMSNorm epsilon: finite and at least 2^-126. The backward forms the
// normalised rows r x in fp32, with r = 1/sqrt(mean(x^2) + eps); this bound
// keeps r <= 2^63, so an all-zero row stays zero there (not inf * 0).
bool eps_in_range(double a) { return std::isfinite(a) && a >= 0x1p-126; }

// The derivative clamp is applied in fp32: it must round to a normal fp32.
bool fp32_normal(double a) {
  const float f = (float)a;
  return std::isfinite(f) && f >= 1.17549435e-38f;
}

// Launch plan for a row of nchunk 16-byte chunks: W waves per row, C chunks
// per thread (FULL when W * 64 * C == nchunk, i.e. no masking), D rows in
// flight per workgroup, weights in LDS (backward), and G workgroups walking
// the rows interleaved (block b takes rows b, b + G, ...). The widths 2048,
// 3072, 4096, 5120, 6144 and 7168 have plans measured on MI355X; other widths
// take the fewest waves that cover the row. G is also the backward's number
// of weight-gradient partials, so it depends only on (T, H).
struct Plan {
  int W, C, D;
  bool full, wlds;
  int64_t blocks;
};

Plan generic_plan(int nchunk) {
  for (int W = 1; W <= 8; W *= 2)
    if (nchunk <= W * kWave) return {W, 1, 2, nchunk == W * kWave, false, 256};
  return {8, 2, 2, nchunk == 8 * kWave * 2, false, 256};
}

// The forward and the backward of one width split the row the same way (same
// W and C), so the backward's recomputed gate has the forward's bits.
Plan fwd_plan(int nchunk) {
  if (nchunk == 896) return {7, 2, 2, true, false, 224};   // H = 7168
  if (nchunk == 512) return {2, 4, 3, true, false, 256};   // H = 4096
  if (nchunk == 640) return {5, 2, 2, true, false, 256};   // H = 5120
  if (nchunk == 384) return {3, 2, 3, true, false, 256};   // H = 3072
  if (nchunk == 256) return {1, 4, 2, true, false, 512};   // H = 2048
  if (nchunk == 768) return {6, 2, 2, true, false, 224};   // H = 6144
  return generic_plan(nchunk);
}

Plan bwd_plan(int nchunk) {
  if (nchunk == 896) return {7, 2, 3, true, true, 224};    // H = 7168
  if (nchunk == 512) return {2, 4, 2, true, false, 256};   // H = 4096
  if (nchunk == 640) return {5, 2, 3, true, true, 256};    // H = 5120
  if (nchunk == 384) return {3, 2, 2, true, false, 256};   // H = 3072
  if (nchunk == 256) return {1, 4, 2, true, false, 512};   // H = 2048
  if (nchunk == 768) return {6, 2, 3, true, true, 224};    // H = 6144
  return generic_plan(nchunk);
}

int64_t grid_of(const Plan& p, int64_t T) { return T < p.blocks ? T : p.blocks; }

// Epochs: each launch of a walk covers at most about kEpochBytes of every
// [T, H] tensor, i.e. at most that many bytes / (G * 2H) rows per block. On
// MI355X a single launch of many rows per block loses bandwidth (the
// backward at H = 7168: 0.73 of 8 TB/s at 16384 rows, 0.70 at 65536 and
// 0.64 at 131072 in one launch; the same rows in launches of 16384 keep
// 0.72-0.73 throughout). 240 MB measured best among 96 to 480 MB.
constexpr int64_t kEpochBytes = (int64_t)240 << 20;

int64_t epoch_iters(int64_t G, int64_t H) {
  const int64_t e = kEpochBytes / (G * H * 2);
  return e > 0 ? e : 1;
}

template <class K>
tk_status launch(K kernel, int grid, int block, void** args, hipStream_t st) {
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid),
                                 dim3(block), args, 0, st);
  return e == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}

struct FwdArgs {
  const u32x4 *x, *k, *v;
  WeightsIn wts;
  u32x4* out;
  float* gate;
  RowWalk walk;
  int nchunk;
  double eps, inv_h, inv_sqrt_h;
};

template <int W, int C, bool FULL, int D, bool FUSED>
tk_status run_fwd(FwdArgs a, int grid, hipStream_t st) {
  void* args[] = {&a.x,    &a.k,    &a.v,      &a.wts, &a.out,
                  &a.gate, &a.walk, &a.nchunk, &a.eps, &a.inv_h, &a.inv_sqrt_h};
  return launch(gate_fwd_kernel<W, C, FULL, D, FUSED>, grid, W * kWave, args, st);
}

template <bool F>
tk_status dispatch_fwd(const Plan& p, const FwdArgs& a, int grid, hipStream_t st) {
  if (p.W == 7 && p.C == 2 && p.full && p.D == 2) return run_fwd<7, 2, true, 2, F>(a, grid, st);
  if (p.W == 2 && p.C == 4 && p.full && p.D == 3) return run_fwd<2, 4, true, 3, F>(a, grid, st);
  if (p.W == 5 && p.C == 2 && p.full && p.D == 2) return run_fwd<5, 2, true, 2, F>(a, grid, st);
  if (p.W == 3 && p.C == 2 && p.full && p.D == 3) return run_fwd<3, 2, true, 3, F>(a, grid, st);
  if (p.W == 1 && p.C == 4 && p.full && p.D == 2) return run_fwd<1, 4, true, 2, F>(a, grid, st);
  if (p.W == 6 && p.C == 2 && p.full && p.D == 2) return run_fwd<6, 2, true, 2, F>(a, grid, st);
  if (p.D == 2 && p.C == 1) {
    switch (p.W) {
      case 1: return run_fwd<1, 1, false, 2, F>(a, grid, st);
      case 2: return run_fwd<2, 1, false, 2, F>(a, grid, st);
      case 4: return run_fwd<4, 1, false, 2, F>(a, grid, st);
      case 8: return run_fwd<8, 1, false, 2, F>(a, grid, st);
      default: break;
    }
  }
  if (p.W == 8 && p.C == 2 && p.D == 2) return run_fwd<8, 2, false, 2, F>(a, grid, st);
  return TK_ERR_UNSUPPORTED;
}

struct BwdArgs {
  const u32x4 *g, *x, *k, *v;
  WeightsIn wts;
  u32x4 *dx, *dk, *dv;
  f32x4* partial;
  RowWalk walk;
  int nchunk;
  double eps, inv_h, inv_sqrt_h;
  float clamp;
  int carry;
};

template <int W, int C, bool FULL, int D, bool WLDS, bool FUSED>
tk_status run_bwd(BwdArgs a, int grid, hipStream_t st) {
  void* args[] = {&a.g,       &a.x,      &a.k,   &a.v,     &a.wts,
                  &a.dx,      &a.dk,     &a.dv,  &a.partial, &a.walk,
                  &a.nchunk,  &a.eps,    &a.clamp, &a.inv_h, &a.inv_sqrt_h,
                  &a.carry};
  return launch(gate_bwd_kernel<W, C, FULL, D, WLDS, FUSED>, grid, W * kWave, args, st);
}

template <bool F>
tk_status dispatch_bwd(const Plan& p, const BwdArgs& a, int grid, hipStream_t st) {
  if (p.W == 7 && p.C == 2 && p.full && p.D == 3 && p.wlds)
    return run_bwd<7, 2, true, 3, true, F>(a, grid, st);
  if (p.W == 2 && p.C == 4 && p.full && p.D == 2 && !p.wlds)
    return run_bwd<2, 4, true, 2, false, F>(a, grid, st);
  if (p.W == 5 && p.C == 2 && p.full && p.D == 3 && p.wlds)
    return run_bwd<5, 2, true, 3, true, F>(a, grid, st);
  if (p.W == 3 && p.C == 2 && p.full && p.D == 2 && !p.wlds)
    return run_bwd<3, 2, true, 2, false, F>(a, grid, st);
  if (p.W == 1 && p.C == 4 && p.full && p.D == 2 && !p.wlds)
    return run_bwd<1, 4, true, 2, false, F>(a, grid, st);
  if (p.W == 6 && p.C == 2 && p.full && p.D == 3 && p.wlds)
    return run_bwd<6, 2, true, 3, true, F>(a, grid, st);
  if (p.D == 2 && !p.wlds && p.C == 1) {
    switch (p.W) {
      case 1: return run_bwd<1, 1, false, 2, false, F>(a, grid, st);
      case 2: return run_bwd<2, 1, false, 2, false, F>(a, grid, st);
      case 4: return run_bwd<4, 1, false, 2, false, F>(a, grid, st);
      case 8: return run_bwd<8, 1, false, 2, false, F>(a, grid, st);
      default: break;
    }
  }
  if (p.W == 8 && p.C == 2 && p.D == 2 && !p.wlds)
    return run_bwd<8, 2, false, 2, false, F>(a, grid, st);
  return TK_ERR_UNSUPPORTED;
}

// The weights as the kernels take them: wh and we, or the fused weight w.
WeightsIn weights_in(const float* wh, const float* we, const double* w) {
  return {reinterpret_cast<const f32x4*>(wh), reinterpret_cast<const f32x4*>(we),
          reinterpret_cast<const f64x2*>(w)};
}

// Argument checks of the forward; w1 and w2 are wh and we, or the fused
// weight twice.
tk_status check_fwd_args(const uint16_t* x, const uint16_t* k, const uint16_t* v,
                         const void* w1, const void* w2, const uint16_t* out,
                         const float* gate, int64_t T, int64_t H, double eps) {
  tk_status st = check_shape(T, H);
  if (st != TK_SUCCESS) return st;
  if (!eps_in_range(eps)) return TK_ERR_VALUE;
  if (T == 0) return TK_SUCCESS;
  if (!x || !k || !v || !w1 || !w2 || !out || !gate) return TK_ERR_NULL;
  if (!aligned16(x) || !aligned16(k) || !aligned16(v) || !aligned16(w1) ||
      !aligned16(w2) || !aligned16(out) || ((uintptr_t)gate & 3u))
    return TK_ERR_ALIGN;
  return TK_SUCCESS;
}

// The forward's launches once its arguments are checked; T > 0.
tk_status enqueue_fwd(const uint16_t* x, const uint16_t* k, const uint16_t* v,
                      WeightsIn wts, uint16_t* out, float* gate, int64_t T, int64_t H,
                      double eps, hipStream_t st) {
  const int nchunk = (int)(H / 8);
  FwdArgs a;
  a.x = reinterpret_cast<const u32x4*>(x);
  a.k = reinterpret_cast<const u32x4*>(k);
  a.v = reinterpret_cast<const u32x4*>(v);
  a.wts = wts;
  a.out = reinterpret_cast<u32x4*>(out);
  a.gate = gate;
  const Plan plan = fwd_plan(nchunk);
  const int grid = (int)grid_of(plan, T);
  a.nchunk = nchunk;
  a.eps = eps;
  a.inv_h = 1.0 / (double)H;
  a.inv_sqrt_h = 1.0 / std::sqrt((double)H);
  const int64_t per_block = (T + grid - 1) / grid;
  const int64_t E = epoch_iters(grid, H);
  a.walk.T = T;
  a.walk.row_step = grid;
  for (int64_t i0 = 0; i0 < per_block; i0 += E) {
    a.walk.iter0 = i0;
    a.walk.iters = std::min(E, per_block - i0);
    const tk_status s =
        wts.w ? dispatch_fwd<true>(plan, a, grid, st) : dispatch_fwd<false>(plan, a, grid, st);
    if (s != TK_SUCCESS) return s;
  }
  return TK_SUCCESS;
}

// Argument checks of the backward (but its workspace); wh and we, or the
// fused weight twice.
tk_status check_bwd_args(const uint16_t* grad_out, const uint16_t* x, const uint16_t* k,
                         const uint16_t* v, const void* wh, const void* we,
                         const uint16_t* dx, const uint16_t* dk, const uint16_t* dv,
                         int64_t T, int64_t H, double eps, double dsqrt_clamp) {
  tk_status st = check_shape(T, H);
  if (st != TK_SUCCESS) return st;
  if (!eps_in_range(eps) || !fp32_normal(dsqrt_clamp)) return TK_ERR_VALUE;
  if (T == 0) return TK_SUCCESS;
  if (!grad_out || !x || !k || !v || !wh || !we || !dx || !dk || !dv) return TK_ERR_NULL;
  if (!aligned16(grad_out) || !aligned16(x) || !aligned16(k) || !aligned16(v) ||
      !aligned16(wh) || !aligned16(we) || !aligned16(dx) || !aligned16(dk) || !aligned16(dv))
    return TK_ERR_ALIGN;
  return TK_SUCCESS;
}

// The backward's launch once its arguments are checked; T > 0.
tk_status enqueue_bwd(const uint16_t* grad_out, const uint16_t* x, const uint16_t* k,
                      const uint16_t* v, WeightsIn wts, uint16_t* dx,
                      uint16_t* dk, uint16_t* dv, float* partial, int64_t T, int64_t H,
                      double eps, double dsqrt_clamp, hipStream_t st) {
  const int nchunk = (int)(H / 8);
  BwdArgs a;
  a.g = reinterpret_cast<const u32x4*>(grad_out);
  a.x = reinterpret_cast<const u32x4*>(x);
  a.k = reinterpret_cast<const u32x4*>(k);
  a.v = reinterpret_cast<const u32x4*>(v);
  a.wts = wts;
  a.dx = reinterpret_cast<u32x4*>(dx);
  a.dk = reinterpret_cast<u32x4*>(dk);
  a.dv = reinterpret_cast<u32x4*>(dv);
  a.partial = reinterpret_cast<f32x4*>(partial);
  const Plan plan = bwd_plan(nchunk);
  const int grid = (int)grid_of(plan, T);
  a.nchunk = nchunk;
  a.eps = eps;
  a.clamp = (float)dsqrt_clamp;
  a.inv_h = 1.0 / (double)H;
  a.inv_sqrt_h = 1.0 / std::sqrt((double)H);
  // the walk in epochs; every epoch after the first continues the partial
  // sums the previous one left in `partial`
  const int64_t per_block = (T + grid - 1) / grid;
  const int64_t E = epoch_iters(grid, H);
  a.walk.T = T;
  a.walk.row_step = grid;
  for (int64_t i0 = 0; i0 < per_block; i0 += E) {
    a.walk.iter0 = i0;
    a.walk.iters = std::min(E, per_block - i0);
    a.carry = i0 > 0;
    const tk_status s =
        wts.w ? dispatch_bwd<true>(plan, a, grid, st) : dispatch_bwd<false>(plan, a, grid, st);
    if (s != TK_SUCCESS) return s;
  }
  return TK_SUCCESS;
}

// The reduction's launch once its arguments are checked.
tk_status enqueue_reduce(const float* workspace, int64_t P, int64_t H, const float* wh,
                         const float* we, float* dwh, float* dwe, hipStream_t st) {
  const f32x4* ws = reinterpret_cast<const f32x4*>(workspace);
  const f32x4* a = reinterpret_cast<const f32x4*>(wh);
  const f32x4* b = reinterpret_cast<const f32x4*>(we);
  f32x4* oh = reinterpret_cast<f32x4*>(dwh);
  f32x4* oe = reinterpret_cast<f32x4*>(dwe);
  int nq = (int)(H / 4);
  void* args[] = {&ws, &P, &nq, &a, &b, &oh, &oe};
  const int grid = (nq + kRedCols4 - 1) / kRedCols4;
  return launch(grad_w_reduce_kernel, grid, kRedCols4 * kRedSlices, args, st);
}

// ---- library-owned partials ---------------------------------------------------

// The weight-gradient partials of tk_engram_gate_bwd_reduce_noalloc live in
// this array: enough for every legal (T, H), P * H <= 256 * 8192 floats
// (8 MiB). Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not the device
// copy, so kernels are given the device address from hipGetSymbolAddress,
// looked up once per device with that device current and kept below.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch[kMaxDevices];

tk_status scratch_of(hipStream_t stream, float** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return TK_ERR_LAUNCH;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return TK_ERR_LAUNCH;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return TK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return TK_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return TK_ERR_LAUNCH;
    if (e != hipSuccess || p == nullptr) return TK_ERR_LAUNCH;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return TK_SUCCESS;
}

}  // namespace

extern "C" {

int64_t tk_engram_num_partials(int64_t T, int64_t H) {
  if (check_shape(T, H) != TK_SUCCESS) return 0;
  return grid_of(bwd_plan((int)(H / 8)), T);
}

int64_t tk_engram_gate_launches(int64_t T, int64_t H, int32_t backward) {
  if (check_shape(T, H) != TK_SUCCESS || T == 0) return 0;
  const int nchunk = (int)(H / 8);
  const int64_t grid = grid_of(backward ? bwd_plan(nchunk) : fwd_plan(nchunk), T);
  const int64_t per_block = (T + grid - 1) / grid;
  const int64_t E = epoch_iters(grid, H);
  return (per_block + E - 1) / E;
}

size_t tk_engram_bwd_workspace_bytes(int64_t T, int64_t H) {
  if (check_shape(T, H) != TK_SUCCESS) return 0;
  return (size_t)tk_engram_num_partials(T, H) * (size_t)H * sizeof(float);
}

tk_status tk_engram_gate_fwd(const uint16_t* x, const uint16_t* k,
                             const uint16_t* v, const float* wh,
                             const float* we, uint16_t* out, float* gate,
                             int64_t T, int64_t H, double eps, void* stream) {
  const tk_status st = check_fwd_args(x, k, v, wh, we, out, gate, T, H, eps);
  if (st != TK_SUCCESS || T == 0) return st;
  return enqueue_fwd(x, k, v, weights_in(wh, we, nullptr), out, gate, T, H, eps,
                     reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_gate_fwd_fused(const uint16_t* x, const uint16_t* k,
                                   const uint16_t* v, const double* w, uint16_t* out,
                                   float* gate, int64_t T, int64_t H, double eps,
                                   void* stream) {
  const tk_status st = check_fwd_args(x, k, v, w, w, out, gate, T, H, eps);
  if (st != TK_SUCCESS || T == 0) return st;
  return enqueue_fwd(x, k, v, weights_in(nullptr, nullptr, w), out, gate, T, H, eps,
                     reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_gate_bwd(const uint16_t* grad_out, const uint16_t* x,
                             const uint16_t* k, const uint16_t* v,
                             const float* wh, const float* we, uint16_t* dx,
                             uint16_t* dk, uint16_t* dv, float* workspace,
                             size_t workspace_bytes, int64_t T, int64_t H,
                             double eps, double dsqrt_clamp, void* stream) {
  tk_status st = check_bwd_args(grad_out, x, k, v, wh, we, dx, dk, dv, T, H, eps, dsqrt_clamp);
  if (st != TK_SUCCESS || T == 0) return st;
  if (!workspace) return TK_ERR_NULL;
  if (!aligned16(workspace)) return TK_ERR_ALIGN;
  if (workspace_bytes < tk_engram_bwd_workspace_bytes(T, H)) return TK_ERR_WORKSPACE;
  return enqueue_bwd(grad_out, x, k, v, weights_in(wh, we, nullptr), dx, dk, dv, workspace,
                     T, H, eps, dsqrt_clamp, reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_gate_bwd_fused(const uint16_t* grad_out, const uint16_t* x,
                                   const uint16_t* k, const uint16_t* v, const double* w,
                                   uint16_t* dx, uint16_t* dk, uint16_t* dv, float* workspace,
                                   size_t workspace_bytes, int64_t T, int64_t H, double eps,
                                   double dsqrt_clamp, void* stream) {
  tk_status st = check_bwd_args(grad_out, x, k, v, w, w, dx, dk, dv, T, H, eps, dsqrt_clamp);
  if (st != TK_SUCCESS || T == 0) return st;
  if (!workspace) return TK_ERR_NULL;
  if (!aligned16(workspace)) return TK_ERR_ALIGN;
  if (workspace_bytes < tk_engram_bwd_workspace_bytes(T, H)) return TK_ERR_WORKSPACE;
  return enqueue_bwd(grad_out, x, k, v, weights_in(nullptr, nullptr, w), dx, dk, dv,
                     workspace, T, H, eps, dsqrt_clamp, reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_grad_w_reduce(const float* workspace, int64_t P, int64_t H,
                                  const float* wh, const float* we, float* dwh,
                                  float* dwe, void* stream) {
  if (P < 0) return TK_ERR_SHAPE;
  tk_status st = check_shape(0, H);
  if (st != TK_SUCCESS) return st;
  if (P > TK_ENGRAM_MAX_PARTIALS) return TK_ERR_UNSUPPORTED;
  if ((P > 0 && !workspace) || !wh || !we || !dwh || !dwe) return TK_ERR_NULL;
  if ((P > 0 && !aligned16(workspace)) || !aligned16(wh) || !aligned16(we) ||
      !aligned16(dwh) || !aligned16(dwe))
    return TK_ERR_ALIGN;
  return enqueue_reduce(workspace, P, H, wh, we, dwh, dwe,
                        reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_gate_bwd_reduce_noalloc(const uint16_t* grad_out, const uint16_t* x,
                                            const uint16_t* k, const uint16_t* v,
                                            const float* wh, const float* we, uint16_t* dx,
                                            uint16_t* dk, uint16_t* dv, float* dwh,
                                            float* dwe, int64_t T, int64_t H, double eps,
                                            double dsqrt_clamp, void* stream) {
  tk_status st = check_bwd_args(grad_out, x, k, v, wh, we, dx, dk, dv, T, H, eps, dsqrt_clamp);
  if (st != TK_SUCCESS) return st;
  // the reduction reads wh and we and writes dwh and dwe even when T = 0
  if (!wh || !we || !dwh || !dwe) return TK_ERR_NULL;
  if (!aligned16(wh) || !aligned16(we) || !aligned16(dwh) || !aligned16(dwe))
    return TK_ERR_ALIGN;
  if (tk_engram_bwd_workspace_bytes(T, H) > sizeof(scratch)) return TK_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  float* partial = nullptr;
  st = scratch_of(hs, &partial);
  if (st != TK_SUCCESS) return st;
  if (T > 0) {
    st = enqueue_bwd(grad_out, x, k, v, weights_in(wh, we, nullptr), dx, dk, dv, partial, T, H,
                     eps, dsqrt_clamp, hs);
    if (st != TK_SUCCESS) return st;
  }
  return enqueue_reduce(partial, tk_engram_num_partials(T, H), H, wh, we, dwh, dwe, hs);
}

tk_status tk_engram_fused_weight(const float* wh, const float* we, double* w, int64_t H,
                                 void* stream) {
  if (H < 0) return TK_ERR_SHAPE;
  if (H == 0) return TK_SUCCESS;
  if (!wh || !we || !w) return TK_ERR_NULL;
  if (((uintptr_t)wh & 3u) || ((uintptr_t)we & 3u) || ((uintptr_t)w & 7u)) return TK_ERR_ALIGN;
  if (H > ((int64_t)1 << 40)) return TK_ERR_UNSUPPORTED;
  const int64_t blocks = (H + 255) / 256;
  void* args[] = {&wh, &we, &w, &H};
  return launch(fused_weight_kernel, (int)blocks, 256, args,
                reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_copy_probe(const void* src, void* dst, size_t bytes,
                               void* stream) {
  if (bytes == 0) return TK_SUCCESS;
  if (!src || !dst) return TK_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst) || (bytes & 15u)) return TK_ERR_ALIGN;
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  int64_t n = (int64_t)(bytes / 16);
  const int64_t tiles = (n + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  const int grid = (int)(tiles < 16384 ? tiles : 16384);
  void* args[] = {&s, &d, &n};
  return launch(copy_probe_kernel, grid, 256, args,
                reinterpret_cast<hipStream_t>(stream));
}

tk_status tk_engram_stream_probe(const void* const* src, int32_t nsrc, void* const* dst,
                                 int32_t ndst, size_t bytes, void* stream) {
  if (nsrc < 1 || ndst < 1 || nsrc > TK_ENGRAM_PROBE_MAX_STREAMS ||
      ndst > TK_ENGRAM_PROBE_MAX_STREAMS)
    return TK_ERR_SHAPE;
  if (!src || !dst) return TK_ERR_NULL;
  if (bytes == 0) return TK_SUCCESS;
  if (bytes & 15u) return TK_ERR_ALIGN;
  StreamSet st = {};
  for (int i = 0; i < nsrc; ++i) {
    if (!src[i]) return TK_ERR_NULL;
    if (!aligned16(src[i])) return TK_ERR_ALIGN;
    st.in[i] = reinterpret_cast<const u32x4*>(src[i]);
  }
  for (int o = 0; o < ndst; ++o) {
    if (!dst[o]) return TK_ERR_NULL;
    if (!aligned16(dst[o])) return TK_ERR_ALIGN;
    st.out[o] = reinterpret_cast<u32x4*>(dst[o]);
  }
  int64_t n = (int64_t)(bytes / 16);
  const int64_t tiles = (n + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  const int grid = (int)(tiles < 32768 ? tiles : 32768);
  void* args[] = {&st, &n};
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
#define TK_PROBE(R, S) \
  if (nsrc == R && ndst == S) return launch(stream_probe_kernel<R, S>, grid, 256, args, hs)
  TK_PROBE(1, 1); TK_PROBE(2, 1); TK_PROBE(3, 1); TK_PROBE(4, 1);
  TK_PROBE(1, 2); TK_PROBE(2, 2); TK_PROBE(3, 2); TK_PROBE(4, 2);
  TK_PROBE(1, 3); TK_PROBE(2, 3); TK_PROBE(3, 3); TK_PROBE(4, 3);
  TK_PROBE(1, 4); TK_PROBE(2, 4); TK_PROBE(3, 4); TK_PROBE(4, 4);
#undef TK_PROBE
  return TK_ERR_UNSUPPORTED;
}

}  // extern "C"
