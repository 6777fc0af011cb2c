// Engram gate for AMD MI355X (gfx950): HIP kernels and the C ABI of
// include/tk_engram.h.
//
// The operation is the gate of the zhichai.net TileKernels page, section
// "5. Engram" (gate formula), with its backward and the weight-gradient
// reduction that the same section lists as separate kernels.
//
// Everything on this path streams bf16 rows from HBM and reduces each row to
// a handful of scalars; nothing is a dense contraction, so no matrix cores
// are used. Each kernel is built around one idea: a workgroup of W waves owns
// a contiguous block of rows and walks it one row at a time; the row is split
// across the W*64 threads in 16-byte chunks (8 bf16), thread `tid` owning
// chunks tid, tid + W*64, ... so that every load and store instruction of a
// wave covers 1 KiB of contiguous memory. While a row is reduced and written,
// the loads of the next row are already in flight.
//
// Algebra used by both passes. With w_i = wh_i * we_i (the product of the
// two RMSNorm weights),
//   d = r_x r_k sum_i x_i k_i w_i,  P = sum_i x_i k_i w_i,
// and the chain rule through out = x + gate * v gives per row
//   dd = (sum_i gout_i v_i) * g (1 - g) / (2 sqrt(max(|z|, clamp))) / sqrt(H)
//   dx_i = gout_i + A w_i k_i - Bx x_i,   dk_i = A w_i x_i - Bk k_i,
//   dv_i = g gout_i,
//   A = dd r_x r_k,  Bx = dd r_x^2 d / H,  Bk = dd r_k^2 d / H,
// and the weight gradients share one column vector c_i = sum_t A_t x_ti k_ti:
//   dL/dwh_i = we_i c_i,   dL/dwe_i = wh_i c_i.
//
// Precision: x_i * k_i is exact in fp32 (two 8-bit significands); it is
// multiplied by w_i and accumulated in fp64, so the dot product that decides
// the gate near z = 0 carries no cancellation error worth the name. The
// sums of squares and of gout*v are fp32; the per-row scalars use the
// hardware's fp32 reciprocal, square root and exp2 (about 1 ulp each), whose
// relative errors move the gate by < 1e-7.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "tk_engram.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// ---- wave reductions (xor butterfly: every lane ends with the same bits) ---

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ---- per-thread slice of a row ---------------------------------------------

// Chunk j of thread `tid` is 16-byte chunk j * NT + tid of the row.
template <int NT, int C, bool FULL>
__device__ __forceinline__ void load_row(const u32x4* __restrict__ row, int tid,
                                         int nchunk, u32x4 (&dst)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    if (FULL || c < nchunk) {
      dst[j] = row[c];
    } else {
      dst[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// w_i = wh_i * we_i for the thread's columns, in fp32 (elementwise work of
// the backward) and exactly in fp64 (the dot product).
template <int NT, int C, bool FULL>
__device__ __forceinline__ void load_weights(const f32x4* __restrict__ wh,
                                             const f32x4* __restrict__ we,
                                             int tid, int nchunk,
                                             float (&w32)[C][8],
                                             double (&w64)[C][8]) {
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = j * NT + tid;
    f32x4 a0 = {0, 0, 0, 0}, a1 = a0, b0 = a0, b1 = a0;
    if (FULL || c < nchunk) {
      a0 = wh[2 * c];
      a1 = wh[2 * c + 1];
      b0 = we[2 * c];
      b1 = we[2 * c + 1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w32[j][e] = a0[e] * b0[e];
      w32[j][e + 4] = a1[e] * b1[e];
      w64[j][e] = (double)a0[e] * (double)b0[e];
      w64[j][e + 4] = (double)a1[e] * (double)b1[e];
    }
  }
}

struct RowScalars {
  float r_x, r_k, d, z, g;
};

// Gate of one row from its three sums (formula of the section "5. Engram").
__device__ __forceinline__ RowScalars row_gate(float sum_xx, float sum_kk,
                                               double sum_xkw, float eps,
                                               float inv_h, float inv_sqrt_h) {
  RowScalars s;
  s.r_x = __builtin_amdgcn_rsqf(fmaf(sum_xx, inv_h, eps));
  s.r_k = __builtin_amdgcn_rsqf(fmaf(sum_kk, inv_h, eps));
  s.d = (float)sum_xkw * s.r_x * s.r_k;
  s.z = s.d * inv_sqrt_h;
  // signed_sqrt: sign(z) sqrt|z|, with sign(0) = 0
  const float sq = copysignf(__builtin_amdgcn_sqrtf(fabsf(s.z)), s.z);
  // sigmoid(sq) = 1 / (1 + 2^(-sq log2 e))
  const float e = __builtin_amdgcn_exp2f(-sq * 1.4426950408889634f);
  s.g = __builtin_amdgcn_rcpf(1.0f + e);
  return s;
}

// ---- forward ---------------------------------------------------------------

template <int W, int C, bool FULL>
__global__ __launch_bounds__(W * kWave) void gate_fwd_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ k,
    const u32x4* __restrict__ v, const f32x4* __restrict__ wh,
    const f32x4* __restrict__ we, u32x4* __restrict__ out,
    float* __restrict__ gate, int64_t T, int nchunk, int64_t rows_per_block,
    float eps, float inv_h, float inv_sqrt_h) {
  constexpr int NT = W * kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  // Per-wave partial sums, double-buffered by row parity so that one barrier
  // per row suffices.
  __shared__ float red_xx[2][W];
  __shared__ float red_kk[2][W];
  __shared__ double red_xkw[2][W];

  float w32[C][8];
  double w64[C][8];
  load_weights<NT, C, FULL>(wh, we, tid, nchunk, w32, w64);

  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);
  if (r0 >= r1) return;

  u32x4 xa[C], ka[C], va[C];
  load_row<NT, C, FULL>(x + r0 * nchunk, tid, nchunk, xa);
  load_row<NT, C, FULL>(k + r0 * nchunk, tid, nchunk, ka);
  load_row<NT, C, FULL>(v + r0 * nchunk, tid, nchunk, va);

  for (int64_t r = r0; r < r1; ++r) {
    const bool more = r + 1 < r1;
    u32x4 xb[C], kb[C], vb[C];
    if (more) {
      const int64_t o = (r + 1) * nchunk;
      load_row<NT, C, FULL>(x + o, tid, nchunk, xb);
      load_row<NT, C, FULL>(k + o, tid, nchunk, kb);
      load_row<NT, C, FULL>(v + o, tid, nchunk, vb);
    }

    float sxx = 0.f, skk = 0.f;
    double sxkw = 0.0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float xf[8], kf[8];
      unpack8(xa[j], xf);
      unpack8(ka[j], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sxx = fmaf(xf[e], xf[e], sxx);
        skk = fmaf(kf[e], kf[e], skk);
        sxkw = fma((double)(xf[e] * kf[e]), w64[j][e], sxkw);
      }
    }
    sxx = wave_sum(sxx);
    skk = wave_sum(skk);
    sxkw = wave_sum(sxkw);
    const int slot = (int)((r - r0) & 1);
    if (lane == 0) {
      red_xx[slot][wave] = sxx;
      red_kk[slot][wave] = skk;
      red_xkw[slot][wave] = sxkw;
    }
    __syncthreads();
    float txx = 0.f, tkk = 0.f;
    double txkw = 0.0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      txx += red_xx[slot][i];
      tkk += red_kk[slot][i];
      txkw += red_xkw[slot][i];
    }
    const RowScalars s = row_gate(txx, tkk, txkw, eps, inv_h, inv_sqrt_h);

    const int64_t o = r * nchunk;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = j * NT + tid;
      if (FULL || c < nchunk) {
        float xf[8], vf[8], of[8];
        unpack8(xa[j], xf);
        unpack8(va[j], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) of[e] = fmaf(s.g, vf[e], xf[e]);
        out[o + c] = pack8(of);
      }
    }
    if (tid == 0) gate[r] = s.g;

    if (more) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        xa[j] = xb[j];
        ka[j] = kb[j];
        va[j] = vb[j];
      }
    }
  }
}

// ---- backward --------------------------------------------------------------

template <int W, int C, bool FULL>
__global__ __launch_bounds__(W * kWave) void gate_bwd_kernel(
    const u32x4* __restrict__ gout, const u32x4* __restrict__ x,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const f32x4* __restrict__ wh, const f32x4* __restrict__ we,
    u32x4* __restrict__ dx, u32x4* __restrict__ dk, u32x4* __restrict__ dv,
    f32x4* __restrict__ partial, int64_t T, int nchunk,
    int64_t rows_per_block, float eps, float clamp, float inv_h,
    float inv_sqrt_h) {
  constexpr int NT = W * kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  __shared__ float red_xx[2][W];
  __shared__ float red_kk[2][W];
  __shared__ float red_gv[2][W];
  __shared__ double red_xkw[2][W];

  float w32[C][8];
  double w64[C][8];
  load_weights<NT, C, FULL>(wh, we, tid, nchunk, w32, w64);

  // c_i over this block's rows, for the thread's columns.
  float cacc[C][8];
#pragma unroll
  for (int j = 0; j < C; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) cacc[j][e] = 0.f;

  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);

  if (r0 < r1) {
    u32x4 ga[C], xa[C], ka[C], va[C];
    load_row<NT, C, FULL>(gout + r0 * nchunk, tid, nchunk, ga);
    load_row<NT, C, FULL>(v + r0 * nchunk, tid, nchunk, va);
    load_row<NT, C, FULL>(x + r0 * nchunk, tid, nchunk, xa);
    load_row<NT, C, FULL>(k + r0 * nchunk, tid, nchunk, ka);

    for (int64_t r = r0; r < r1; ++r) {
      const bool more = r + 1 < r1;
      u32x4 gb[C], xb[C], kb[C], vb[C];
      if (more) {
        const int64_t o = (r + 1) * nchunk;
        load_row<NT, C, FULL>(gout + o, tid, nchunk, gb);
        load_row<NT, C, FULL>(v + o, tid, nchunk, vb);
        load_row<NT, C, FULL>(x + o, tid, nchunk, xb);
        load_row<NT, C, FULL>(k + o, tid, nchunk, kb);
      }

      float sxx = 0.f, skk = 0.f, sgv = 0.f;
      double sxkw = 0.0;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        float gf[8], xf[8], kf[8], vf[8];
        unpack8(ga[j], gf);
        unpack8(va[j], vf);
        unpack8(xa[j], xf);
        unpack8(ka[j], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sgv = fmaf(gf[e], vf[e], sgv);
          sxx = fmaf(xf[e], xf[e], sxx);
          skk = fmaf(kf[e], kf[e], skk);
          sxkw = fma((double)(xf[e] * kf[e]), w64[j][e], sxkw);
        }
      }
      sxx = wave_sum(sxx);
      skk = wave_sum(skk);
      sgv = wave_sum(sgv);
      sxkw = wave_sum(sxkw);
      const int slot = (int)((r - r0) & 1);
      if (lane == 0) {
        red_xx[slot][wave] = sxx;
        red_kk[slot][wave] = skk;
        red_gv[slot][wave] = sgv;
        red_xkw[slot][wave] = sxkw;
      }
      __syncthreads();
      float txx = 0.f, tkk = 0.f, tgv = 0.f;
      double txkw = 0.0;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        txx += red_xx[slot][i];
        tkk += red_kk[slot][i];
        tgv += red_gv[slot][i];
        txkw += red_xkw[slot][i];
      }
      const RowScalars s = row_gate(txx, tkk, txkw, eps, inv_h, inv_sqrt_h);
      // gate = sigmoid(sq): d gate / d sq = g (1 - g);
      // sq = signed_sqrt(z): d sq / dz = 1 / (2 sqrt(max(|z|, clamp)));
      // z = d / sqrt(H).
      const float ds = tgv * s.g * (1.0f - s.g);
      const float dz = ds * 0.5f * __builtin_amdgcn_rsqf(fmaxf(fabsf(s.z), clamp));
      const float dd = dz * inv_sqrt_h;
      const float A = dd * s.r_x * s.r_k;
      const float Bx = dd * s.r_x * s.r_x * s.d * inv_h;
      const float Bk = dd * s.r_k * s.r_k * s.d * inv_h;

      const int64_t o = r * nchunk;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int c = j * NT + tid;
        if (FULL || c < nchunk) {
          float gf[8], xf[8], kf[8], ox[8], ok[8], ov[8];
          unpack8(ga[j], gf);
          unpack8(xa[j], xf);
          unpack8(ka[j], kf);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ox[e] = fmaf(-Bx, xf[e], fmaf(A, w32[j][e] * kf[e], gf[e]));
            ok[e] = fmaf(-Bk, kf[e], A * (w32[j][e] * xf[e]));
            ov[e] = s.g * gf[e];
            cacc[j][e] = fmaf(A, xf[e] * kf[e], cacc[j][e]);
          }
          dx[o + c] = pack8(ox);
          dk[o + c] = pack8(ok);
          dv[o + c] = pack8(ov);
        }
      }

      if (more) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
          ga[j] = gb[j];
          xa[j] = xb[j];
          ka[j] = kb[j];
          va[j] = vb[j];
        }
      }
    }
  }

  // This block's partial row of c.
  f32x4* prow = partial + (int64_t)blockIdx.x * (2 * nchunk);
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

// 256 threads: 16 groups of 4 columns x 16 strided slices of the partials.
// Each thread sums its slice in increasing p; the 16 slice sums are then
// added in increasing slice order. The order depends only on (P, H).
constexpr int kRedCols4 = 16;
constexpr int kRedSlices = 16;

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
    for (int64_t p = py; p < P; p += kRedSlices) s += partial[p * nq + q];
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

// ---- copy probe ------------------------------------------------------------

__global__ __launch_bounds__(256) void copy_probe_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
          d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// ---- host side -------------------------------------------------------------

// Target number of row blocks; each block reduces its rows' weight-gradient
// contribution into one partial row.
constexpr int64_t kTargetBlocks = 512;

int64_t rows_per_block(int64_t T) {
  if (T <= 0) return 1;
  return (T + kTargetBlocks - 1) / kTargetBlocks;
}

int64_t num_blocks(int64_t T) {
  if (T <= 0) return 0;
  const int64_t rpb = rows_per_block(T);
  return (T + rpb - 1) / rpb;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

tk_status check_shape(int64_t T, int64_t H) {
  if (T < 0 || H <= 0) return TK_ERR_SHAPE;
  if (H % 8 != 0) return TK_ERR_ALIGN;
  if (H > TK_ENGRAM_MAX_H) return TK_ERR_UNSUPPORTED;
  return TK_SUCCESS;
}

bool finite_positive(double a) { return std::isfinite(a) && a > 0.0; }

// Launch shape for a row of nchunk 16-byte chunks: W waves, C chunks per
// thread; FULL when W * 64 * C == nchunk exactly (no masking).
struct Shape {
  int W, C;
  bool full;
};

Shape pick_shape(int nchunk) {
  if (nchunk == 896) return {7, 2, true};   // H = 7168
  if (nchunk == 512) return {4, 2, true};   // H = 4096
  // Other widths: the fewest waves (1..8) that cover the row with one chunk
  // per thread, else 8 waves with two; trailing chunks may be masked.
  for (int W = 1; W <= 8; W *= 2)
    if (nchunk <= W * kWave) return {W, 1, nchunk == W * kWave};
  return {8, 2, nchunk == 8 * kWave * 2};
}

template <class K>
tk_status launch(K kernel, int grid, int block, void** args, hipStream_t st) {
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid),
                                 dim3(block), args, 0, st);
  return e == hipSuccess ? TK_SUCCESS : TK_ERR_LAUNCH;
}

struct FwdArgs {
  const u32x4 *x, *k, *v;
  const f32x4 *wh, *we;
  u32x4* out;
  float* gate;
  int64_t T;
  int nchunk;
  int64_t rpb;
  float eps, inv_h, inv_sqrt_h;
};

template <int W, int C, bool FULL>
tk_status run_fwd(FwdArgs a, int grid, hipStream_t st) {
  void* args[] = {&a.x, &a.k, &a.v, &a.wh, &a.we, &a.out, &a.gate, &a.T,
                  &a.nchunk, &a.rpb, &a.eps, &a.inv_h, &a.inv_sqrt_h};
  return launch(gate_fwd_kernel<W, C, FULL>, grid, W * kWave, args, st);
}

struct BwdArgs {
  const u32x4 *g, *x, *k, *v;
  const f32x4 *wh, *we;
  u32x4 *dx, *dk, *dv;
  f32x4* partial;
  int64_t T;
  int nchunk;
  int64_t rpb;
  float eps, clamp, inv_h, inv_sqrt_h;
};

template <int W, int C, bool FULL>
tk_status run_bwd(BwdArgs a, int grid, hipStream_t st) {
  void* args[] = {&a.g,  &a.x,       &a.k,      &a.v,   &a.wh,    &a.we,
                  &a.dx, &a.dk,      &a.dv,     &a.partial, &a.T, &a.nchunk,
                  &a.rpb, &a.eps,    &a.clamp,  &a.inv_h, &a.inv_sqrt_h};
  return launch(gate_bwd_kernel<W, C, FULL>, grid, W * kWave, args, st);
}

// Dispatch over the instantiated shapes. Returns TK_ERR_UNSUPPORTED if the
// shape picked does not cover the row (cannot happen for H <= 8192).
#define TK_DISPATCH(RUN, ARGS, GRID, ST, SHAPE)                                 \
  do {                                                                          \
    const Shape s_ = (SHAPE);                                                   \
    if (s_.W == 7 && s_.C == 2 && s_.full) return RUN<7, 2, true>(ARGS, GRID, ST); \
    if (s_.W == 4 && s_.C == 2 && s_.full) return RUN<4, 2, true>(ARGS, GRID, ST); \
    if (s_.C == 1) {                                                            \
      switch (s_.W) {                                                           \
        case 1: return RUN<1, 1, false>(ARGS, GRID, ST);                        \
        case 2: return RUN<2, 1, false>(ARGS, GRID, ST);                        \
        case 4: return RUN<4, 1, false>(ARGS, GRID, ST);                        \
        case 8: return RUN<8, 1, false>(ARGS, GRID, ST);                        \
        default: break;                                                         \
      }                                                                         \
    }                                                                           \
    if (s_.W == 8 && s_.C == 2) return RUN<8, 2, false>(ARGS, GRID, ST);       \
    return TK_ERR_UNSUPPORTED;                                                  \
  } while (0)

}  // namespace

extern "C" {

int32_t tk_abi_version(void) { return TK_ENGRAM_ABI_VERSION; }

const char* tk_status_string(tk_status s) {
  switch (s) {
    case TK_SUCCESS: return "success";
    case TK_ERR_NULL: return "a required pointer is NULL";
    case TK_ERR_SHAPE: return "invalid shape (T < 0, H <= 0 or P < 0)";
    case TK_ERR_ALIGN: return "H is not a multiple of 8 or a pointer is not 16-byte aligned";
    case TK_ERR_UNSUPPORTED: return "H exceeds the supported maximum (8192)";
    case TK_ERR_WORKSPACE: return "backward workspace is smaller than required";
    case TK_ERR_LAUNCH: return "kernel launch failed";
    case TK_ERR_VALUE: return "eps or clamp is not a finite positive number";
    default: return "unknown status";
  }
}

int64_t tk_engram_num_partials(int64_t T, int64_t H) {
  if (check_shape(T, H) != TK_SUCCESS) return 0;
  return num_blocks(T);
}

size_t tk_engram_bwd_workspace_bytes(int64_t T, int64_t H) {
  if (check_shape(T, H) != TK_SUCCESS) return 0;
  return (size_t)num_blocks(T) * (size_t)H * sizeof(float);
}

tk_status tk_engram_gate_fwd(const uint16_t* x, const uint16_t* k,
                             const uint16_t* v, const float* wh,
                             const float* we, uint16_t* out, float* gate,
                             int64_t T, int64_t H, double eps, void* stream) {
  tk_status st = check_shape(T, H);
  if (st != TK_SUCCESS) return st;
  if (!finite_positive(eps)) return TK_ERR_VALUE;
  if (T == 0) return TK_SUCCESS;
  if (!x || !k || !v || !wh || !we || !out || !gate) return TK_ERR_NULL;
  if (!aligned16(x) || !aligned16(k) || !aligned16(v) || !aligned16(wh) ||
      !aligned16(we) || !aligned16(out) || ((uintptr_t)gate & 3u))
    return TK_ERR_ALIGN;
  const int nchunk = (int)(H / 8);
  FwdArgs a;
  a.x = reinterpret_cast<const u32x4*>(x);
  a.k = reinterpret_cast<const u32x4*>(k);
  a.v = reinterpret_cast<const u32x4*>(v);
  a.wh = reinterpret_cast<const f32x4*>(wh);
  a.we = reinterpret_cast<const f32x4*>(we);
  a.out = reinterpret_cast<u32x4*>(out);
  a.gate = gate;
  a.T = T;
  a.nchunk = nchunk;
  a.rpb = rows_per_block(T);
  a.eps = (float)eps;
  a.inv_h = (float)(1.0 / (double)H);
  a.inv_sqrt_h = (float)(1.0 / std::sqrt((double)H));
  const int grid = (int)num_blocks(T);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  TK_DISPATCH(run_fwd, a, grid, hs, pick_shape(nchunk));
}

tk_status tk_engram_gate_bwd(const uint16_t* grad_out, const uint16_t* x,
                             const uint16_t* k, const uint16_t* v,
                             const float* wh, const float* we, uint16_t* dx,
                             uint16_t* dk, uint16_t* dv, float* workspace,
                             size_t workspace_bytes, int64_t T, int64_t H,
                             double eps, double dsqrt_clamp, void* stream) {
  tk_status st = check_shape(T, H);
  if (st != TK_SUCCESS) return st;
  if (!finite_positive(eps) || !finite_positive(dsqrt_clamp)) return TK_ERR_VALUE;
  if (T == 0) return TK_SUCCESS;
  if (!grad_out || !x || !k || !v || !wh || !we || !dx || !dk || !dv || !workspace)
    return TK_ERR_NULL;
  if (!aligned16(grad_out) || !aligned16(x) || !aligned16(k) || !aligned16(v) ||
      !aligned16(wh) || !aligned16(we) || !aligned16(dx) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace))
    return TK_ERR_ALIGN;
  if (workspace_bytes < tk_engram_bwd_workspace_bytes(T, H)) return TK_ERR_WORKSPACE;
  const int nchunk = (int)(H / 8);
  BwdArgs a;
  a.g = reinterpret_cast<const u32x4*>(grad_out);
  a.x = reinterpret_cast<const u32x4*>(x);
  a.k = reinterpret_cast<const u32x4*>(k);
  a.v = reinterpret_cast<const u32x4*>(v);
  a.wh = reinterpret_cast<const f32x4*>(wh);
  a.we = reinterpret_cast<const f32x4*>(we);
  a.dx = reinterpret_cast<u32x4*>(dx);
  a.dk = reinterpret_cast<u32x4*>(dk);
  a.dv = reinterpret_cast<u32x4*>(dv);
  a.partial = reinterpret_cast<f32x4*>(workspace);
  a.T = T;
  a.nchunk = nchunk;
  a.rpb = rows_per_block(T);
  a.eps = (float)eps;
  a.clamp = (float)dsqrt_clamp;
  a.inv_h = (float)(1.0 / (double)H);
  a.inv_sqrt_h = (float)(1.0 / std::sqrt((double)H));
  const int grid = (int)num_blocks(T);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  TK_DISPATCH(run_bwd, a, grid, hs, pick_shape(nchunk));
}

tk_status tk_engram_grad_w_reduce(const float* workspace, int64_t P, int64_t H,
                                  const float* wh, const float* we, float* dwh,
                                  float* dwe, void* stream) {
  if (P < 0) return TK_ERR_SHAPE;
  tk_status st = check_shape(0, H);
  if (st != TK_SUCCESS) return st;
  if ((P > 0 && !workspace) || !wh || !we || !dwh || !dwe) return TK_ERR_NULL;
  if ((P > 0 && !aligned16(workspace)) || !aligned16(wh) || !aligned16(we) ||
      !aligned16(dwh) || !aligned16(dwe))
    return TK_ERR_ALIGN;
  const f32x4* ws = reinterpret_cast<const f32x4*>(workspace);
  const f32x4* a = reinterpret_cast<const f32x4*>(wh);
  const f32x4* b = reinterpret_cast<const f32x4*>(we);
  f32x4* oh = reinterpret_cast<f32x4*>(dwh);
  f32x4* oe = reinterpret_cast<f32x4*>(dwe);
  int nq = (int)(H / 4);
  void* args[] = {&ws, &P, &nq, &a, &b, &oh, &oe};
  const int grid = (nq + kRedCols4 - 1) / kRedCols4;
  return launch(grad_w_reduce_kernel, grid, kRedCols4 * kRedSlices, args,
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
  int64_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 8192 ? blocks : 8192);
  void* args[] = {&s, &d, &n};
  return launch(copy_probe_kernel, grid, 256, args,
                reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
