/*
 * tk_engram.h — C ABI of the Engram gate library for AMD MI355X (gfx950).
 *
 * The operation is the Engram gate of DeepSeek's TileKernels as described on
 * the zhichai.net TileKernels page, section "5. Engram" (gate formula). Per
 * token (row) t, with x the hidden row (the formula's hidden_states), k the
 * key row, v the value row, all of width H, and per-channel RMSNorm weights
 * wh and we:
 *
 *   r_x    = 1 / sqrt(mean(x^2) + eps)      RMSNorm(x, wh) = x * r_x * wh
 *   r_k    = 1 / sqrt(mean(k^2) + eps)      RMSNorm(k, we) = k * r_k * we
 *   d      = dot(RMSNorm(x, wh), RMSNorm(k, we))
 *   z      = d / sqrt(H)                    (the formula's scalar)
 *   gate   = sigmoid(sign(z) * sqrt(|z|))   (signed_sqrt, then sigmoid)
 *   out    = x + gate * v
 *
 * The same section splits the work into a fused forward, its backward and a
 * separate weight-gradient reduction; the juejin.cn page (highlight 5) says
 * the PyTorch binding covers forward, backward and weight-gradient
 * reduction. The three calls below are that split.
 *
 * Conventions shared by every call:
 *   - Tensors are row-major and contiguous. bf16 tensors cross the ABI as
 *     uint16_t bit patterns; [T, H] means row stride H elements.
 *   - All tensor pointers are DEVICE pointers owned by the caller; the hash,
 *     the gather and the stream probe also take small HOST arrays (of
 *     parameters or of device pointers), read before the call returns, as
 *     stated with each call. No call allocates, frees or synchronises;
 *     each call only enqueues work on `stream` (a hipStream_t passed as
 *     void*, NULL = default stream) and returns. Outputs are overwritten,
 *     never accumulated into. The one piece of library-owned device memory
 *     is the static array of tk_engram_gate_bwd_reduce_noalloc, which the
 *     HIP runtime places on each GPU with the library's code.
 *   - Inputs and outputs must not overlap (undefined behaviour otherwise).
 *   - Arithmetic: every row sum (squares, the weighted dot product
 *     sum_i x_i k_i wh_i we_i, and sum_i grad_out_i v_i) is accumulated in
 *     fp64 from exact products, and the per-row scalars are fp64; the
 *     elementwise work is fp32 on the RMS-normalised rows. So the gate stays
 *     accurate where the dot product is near zero, and no finite bf16 input,
 *     however large or small, overflows or underflows on the way (only
 *     outputs beyond the bf16 range are infinite, as their exact values
 *     would round). bf16 results are rounded to nearest, ties to even.
 *   - Every call is deterministic: the row-to-workgroup assignment depends
 *     only on (T, H), and no atomics are used, so reruns are bit-identical.
 *   - Errors: arguments are checked before any device work; a failed check
 *     returns its status and enqueues nothing. A launch failure returns
 *     TK_ERR_LAUNCH (a call of several launches leaves the ones before it
 *     enqueued). Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - The gate calls walk long batches in several launches (epochs of about
 *     240 MB of each [T, H] tensor) on `stream`; the split depends only on
 *     (T, H) and does not change any result bit.
 *   - Shape limits of the gate calls: 0 <= T, 8 <= H <= 8192, H a multiple
 *     of 8; T = 0 is a successful no-op. The hash and the gather state
 *     their own limits below.
 *   - Alignment: every tensor pointer of the gate calls must be 16-byte
 *     aligned (128-bit loads and stores), except `gate` which needs 4 bytes;
 *     the other calls state their own alignment.
 */
#ifndef TK_ENGRAM_H
#define TK_ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tk_status;

enum {
  TK_SUCCESS = 0,
  TK_ERR_NULL = 1,        /* a required pointer is NULL                     */
  TK_ERR_SHAPE = 2,       /* negative count, width or table count <= 0     */
  TK_ERR_ALIGN = 3,       /* width not a multiple of 8, pointer misaligned */
  TK_ERR_UNSUPPORTED = 4, /* a size above the call's supported maximum      */
  TK_ERR_WORKSPACE = 5,   /* backward workspace smaller than required       */
  TK_ERR_LAUNCH = 6,      /* the HIP runtime refused the kernel launch      */
  TK_ERR_VALUE = 7        /* a scalar or table parameter is out of range    */
};

#define TK_ENGRAM_ABI_VERSION 1
#define TK_ENGRAM_MAX_H 8192
/* Largest number of weight-gradient partial rows any (T, H) uses. */
#define TK_ENGRAM_MAX_PARTIALS 512

/*
 * Forward: zhichai.net TileKernels page, section "5. Engram", gate formula
 * (engram_gate_fwd fuses RMSNorm, signed-sqrt and the sigmoid gate).
 *
 *   x, k, v : bf16 [T, H]  inputs (x is the formula's hidden_states)
 *   wh, we  : fp32 [H]     RMSNorm weights of x and of k
 *   out     : bf16 [T, H]  out = x + gate * v
 *   gate    : fp32 [T]     the gate of each token
 *   eps     : RMSNorm epsilon (inside the square root), finite and at least
 *             2^-126 (FLT_MIN), else TK_ERR_VALUE: the backward forms the
 *             normalised rows 1/sqrt(mean + eps) * x in fp32, and the bound
 *             keeps that scale finite (at most 2^63) for all-zero rows
 */
tk_status tk_engram_gate_fwd(const uint16_t* x, const uint16_t* k,
                             const uint16_t* v, const float* wh,
                             const float* we, uint16_t* out, float* gate,
                             int64_t T, int64_t H, double eps, void* stream);

/*
 * Number of weight-gradient partial rows P the backward writes for (T, H):
 * partial row p sums the tokens t = p, p + P, p + 2P, ... (one workgroup
 * each). A pure function of (T, H), at most T; 0 when T = 0.
 */
int64_t tk_engram_num_partials(int64_t T, int64_t H);

/*
 * Number of kernel launches tk_engram_gate_fwd (backward = 0) or
 * tk_engram_gate_bwd (backward != 0), and their _fused forms, enqueue for
 * (T, H): the row walk split into epochs of about 240 MB of each [T, H]
 * tensor. A pure function of (T, H); 0 when T = 0 or the shape is invalid.
 */
int64_t tk_engram_gate_launches(int64_t T, int64_t H, int32_t backward);

/* Bytes of backward workspace needed for (T, H): P * H * sizeof(float). */
size_t tk_engram_bwd_workspace_bytes(int64_t T, int64_t H);

/*
 * Backward of the forward above (section "5. Engram": engram_gate_bwd), by
 * the chain rule through out = x + gate * v, the sigmoid, signed_sqrt, the
 * scalar, the dot product and both RMSNorms.
 *
 *   grad_out        : bf16 [T, H]  dL/d out
 *   x, k, v, wh, we : as for the forward
 *   dx, dk, dv      : bf16 [T, H]  dL/dx, dL/dk, dL/dv
 *   workspace       : fp32 [P, H]  weight-gradient partials
 *                     c_p[i] = sum over the tokens t = p, p + P, ... of
 *                              dd_t * r_x,t * r_k,t * x_t,i * k_t,i
 *                     with dd_t = dL/dd_t; input to tk_engram_grad_w_reduce
 *   workspace_bytes : size of `workspace`, at least
 *                     tk_engram_bwd_workspace_bytes(T, H)
 *   eps             : as for the forward
 *   dsqrt_clamp     : the derivative of signed_sqrt, 1 / (2 sqrt|z|), is
 *                     evaluated as 1 / (2 sqrt(max(|z|, dsqrt_clamp))) so it
 *                     stays finite at z = 0 (the page gives no value there);
 *                     it is applied in fp32, so it must round to a normal
 *                     positive fp32 value (2^-126 .. FLT_MAX), else
 *                     TK_ERR_VALUE
 *
 * The gate is recomputed from x and k with the forward's arithmetic and
 * summation order, so it has the forward's bits and dv = bf16(gate * grad_out)
 * with the forward's fp32 gate.
 */
tk_status tk_engram_gate_bwd(const uint16_t* grad_out, const uint16_t* x,
                             const uint16_t* k, const uint16_t* v,
                             const float* wh, const float* we, uint16_t* dx,
                             uint16_t* dk, uint16_t* dv, float* workspace,
                             size_t workspace_bytes, int64_t T, int64_t H,
                             double eps, double dsqrt_clamp, void* stream);

/*
 * Weight-gradient reduction (section "5. Engram": engram_grad_w_reduce): a
 * fixed-order tree over the P partial rows written by tk_engram_gate_bwd,
 *   c[i]   = sum_p workspace[p, i]
 *   dwh[i] = we[i] * c[i]      (dL/dwh)
 *   dwe[i] = wh[i] * c[i]      (dL/dwe)
 * since dL/dwh_i = sum_t dd_t r_x,t x_t,i * (r_k,t k_t,i we_i) and likewise
 * for we. P = 0 writes zeros.
 *
 *   workspace : fp32 [P, H], P = tk_engram_num_partials(T, H); the call has
 *               no size argument, so it trusts the caller that the buffer
 *               holds P * H values
 *   P         : 0 .. TK_ENGRAM_MAX_PARTIALS, else TK_ERR_UNSUPPORTED
 *   wh, we    : fp32 [H]
 *   dwh, dwe  : fp32 [H]
 */
tk_status tk_engram_grad_w_reduce(const float* workspace, int64_t P, int64_t H,
                                  const float* wh, const float* we, float* dwh,
                                  float* dwe, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * backward and the weight-gradient reduction in one call, with the
 * weight-gradient partials kept in library-owned device memory instead of a
 * caller's workspace. Its results are those of tk_engram_gate_bwd followed
 * by tk_engram_grad_w_reduce, bit for bit (the same kernels and the same P).
 *
 *   grad_out, x, k, v, wh, we, dx, dk, dv, eps, dsqrt_clamp : as for
 *                     tk_engram_gate_bwd
 *   dwh, dwe        : fp32 [H], as for tk_engram_grad_w_reduce
 *
 * The partials live in a static device array of
 * TK_ENGRAM_NOALLOC_SCRATCH_BYTES (8 MiB), enough for every (T, H) the gate
 * calls accept; a shape needing more returns TK_ERR_WORKSPACE. Each GPU the
 * library runs on holds its own copy until the process ends; its address is
 * looked up once per device (hipGetSymbolAddress), on the first call there,
 * so make that first call (T = 0 will do) before capturing a HIP graph. The
 * call allocates nothing and writes no memset. Every call on one GPU shares that GPU's
 * array, which keeps the last call's partials: the backward writes every
 * partial it uses, so nothing needs clearing, but calls that overlap on one
 * GPU (two streams in flight at once) race and must be serialised by the
 * caller. T = 0 writes zeros to dwh and dwe (wh, we, dwh and dwe are
 * checked then too, since the reduction still runs).
 */
#define TK_ENGRAM_NOALLOC_SCRATCH_BYTES (256u * 8192u * 4u)

tk_status tk_engram_gate_bwd_reduce_noalloc(const uint16_t* grad_out, const uint16_t* x,
                                            const uint16_t* k, const uint16_t* v,
                                            const float* wh, const float* we, uint16_t* dx,
                                            uint16_t* dk, uint16_t* dv, float* dwh,
                                            float* dwe, int64_t T, int64_t H, double eps,
                                            double dsqrt_clamp, void* stream);

/*
 * Fused RMSNorm weight (section "5. Engram": engram_fused_weight, the weight
 * preprocessing step). The two RMSNorm weights enter the gate only through
 * their product, since dot(RMSNorm(x, wh), RMSNorm(k, we)) =
 * r_x * r_k * sum_i x_i k_i (wh_i * we_i); this call forms that product,
 *
 *   w[i] = wh[i] * we[i]    in fp64, exactly (a product of two fp32 values)
 *
 *   wh, we : fp32 [H], device, 4-byte aligned
 *   w      : fp64 [H], device, 8-byte aligned
 *
 * tk_engram_gate_fwd_fused and tk_engram_gate_bwd_fused below take w in
 * place of wh and we; tk_engram_gate_fwd and tk_engram_gate_bwd form the same
 * exact products themselves (O(H) per launch). H = 0 is a successful no-op.
 */
tk_status tk_engram_fused_weight(const float* wh, const float* we, double* w, int64_t H,
                                 void* stream);

/*
 * The forward and the backward with the fused RMSNorm weight (section
 * "5. Engram": engram_fused_weight, then the gate): w = wh * we, fp64 [H],
 * device, 16-byte aligned, in place of wh and we; every other argument,
 * limit and error as for tk_engram_gate_fwd and tk_engram_gate_bwd. With w
 * from tk_engram_fused_weight(wh, we) the results are those of the unfused
 * calls bit for bit: the unfused kernels form exactly this w. The
 * weight-gradient reduction still needs wh and we separately (dL/dwh = we *
 * c, dL/dwe = wh * c), so it takes them as before. For any other fp64 w the
 * calls compute the gate with that weight product; the elementwise backward
 * rounds it to fp32.
 */
tk_status tk_engram_gate_fwd_fused(const uint16_t* x, const uint16_t* k,
                                   const uint16_t* v, const double* w, uint16_t* out,
                                   float* gate, int64_t T, int64_t H, double eps,
                                   void* stream);

tk_status tk_engram_gate_bwd_fused(const uint16_t* grad_out, const uint16_t* x,
                                   const uint16_t* k, const uint16_t* v, const double* w,
                                   uint16_t* dx, uint16_t* dk, uint16_t* dv, float* workspace,
                                   size_t workspace_bytes, int64_t T, int64_t H, double eps,
                                   double dsqrt_clamp, void* stream);

/*
 * N-gram hash of the Engram memory (section "5. Engram": engram_hash, the
 * step before the gate: N-gram token ids combined by XOR and multiplication
 * and mapped to embedding-table indices; the page describes 2 N-gram layers,
 * N up to 3, and 8 tables per layer). The page gives no constants, so the
 * multipliers and table sizes are the caller's. For sequence b, position s,
 * layer l and table j of that layer:
 *
 *   h   = XOR over i < ngram[l] of ( tok(b, s - i) * mult[l][j][i]  mod 2^64 )
 *   out[b][s][l][j] = h mod table_size[l][j]
 *
 * where tok(b, p) is tokens[b][p] taken as an unsigned 32-bit pattern, and
 * `pad` for p < 0 (before the start of the sequence).
 *
 *   tokens     : int32 [B, S], device, 4-byte aligned
 *   ngram      : int32 [L], HOST, each in 1 .. TK_ENGRAM_HASH_MAX_NGRAM
 *   mult       : uint64 [L, K, TK_ENGRAM_HASH_MAX_NGRAM], HOST (entries
 *                i >= ngram[l] are ignored)
 *   table_size : uint32 [L, K], HOST, each in 1 .. TK_ENGRAM_HASH_MAX_TABLE_SIZE
 *   out        : int32 [B, S, L, K], device, 16-byte aligned
 *
 * Limits: L, K >= 1, L * K <= TK_ENGRAM_HASH_MAX_TABLES, B <=
 * TK_ENGRAM_HASH_MAX_BATCH. The host arrays are read during the call only.
 * B = 0 or S = 0 is a successful no-op. Exact integer arithmetic: results are
 * bit-identical to any correct implementation of the formula above.
 */
#define TK_ENGRAM_HASH_MAX_TABLES 32
#define TK_ENGRAM_HASH_MAX_NGRAM 4
#define TK_ENGRAM_HASH_MAX_TABLE_SIZE 2147483648u
#define TK_ENGRAM_HASH_MAX_BATCH 65535

tk_status tk_engram_hash(const int32_t* tokens, int64_t B, int64_t S, int32_t L,
                         int32_t K, const int32_t* ngram, const uint64_t* mult,
                         const uint32_t* table_size, uint32_t pad, int32_t* out,
                         void* stream);

/*
 * Hashed multi-table gather (section "5. Engram": the N-gram hashed embedding
 * tables with O(1) retrieval that tk_engram_hash indexes). The Q tables are
 * packed in one bf16 buffer; table q holds rows [row_offset[q],
 * row_offset[q] + rows[q]). For token t and table q:
 *
 *   out[t][q][:] = table_data[row_offset[q] + idx[t][q]][:]   if 0 <= idx[t][q] < rows[q]
 *   out[t][q][:] = 0                                          otherwise
 *
 *   idx        : int32 [T, Q], device, 4-byte aligned (e.g. tk_engram_hash's
 *                output with Q = L * K)
 *   table_data : bf16 [total_rows, d], device, 16-byte aligned
 *   row_offset : int64 [Q], HOST; rows : uint32 [Q], HOST; every table must
 *                lie inside [0, total_rows)
 *   out        : bf16 [T, Q, d], device, 16-byte aligned
 *
 * Limits: 1 <= Q <= TK_ENGRAM_GATHER_MAX_TABLES, d a multiple of 8 and at
 * most TK_ENGRAM_GATHER_MAX_D, T < 2^31. T = 0 is a successful no-op. Every
 * index is checked against its table on the device, so no index value reads
 * outside the buffer. An exact copy: results are bit-identical to any
 * correct gather.
 */
#define TK_ENGRAM_GATHER_MAX_TABLES 32
#define TK_ENGRAM_GATHER_MAX_D 8192

tk_status tk_engram_gather(const int32_t* idx, int64_t T, int32_t Q,
                           const uint16_t* table_data, int64_t total_rows, int64_t d,
                           const int64_t* row_offset, const uint32_t* rows,
                           uint16_t* out, void* stream);

/*
 * Measurement aid, not part of the gate: copies `bytes` bytes (a multiple
 * of 16, both pointers 16-byte aligned) with the same 128-bit access width
 * as the gate kernels, to calibrate hardware byte counters and to give the
 * practical HBM ceiling of the device it runs on.
 */
tk_status tk_engram_copy_probe(const void* src, void* dst, size_t bytes,
                               void* stream);

/*
 * Measurement aid, not part of the gate: streams nsrc input buffers and
 * writes ndst output buffers of `bytes` bytes each (a multiple of 16, every
 * pointer 16-byte aligned; src and dst are HOST arrays of device pointers),
 * output o being the XOR of all inputs plus o, in the same tiled
 * nontemporal pattern as tk_engram_copy_probe. It gives the practical HBM
 * ceiling of a kernel's read/write mix: 3 in / 1 out for the forward, 4 in /
 * 3 out for the backward. 1 <= nsrc, ndst <= TK_ENGRAM_PROBE_MAX_STREAMS.
 */
#define TK_ENGRAM_PROBE_MAX_STREAMS 4

tk_status tk_engram_stream_probe(const void* const* src, int32_t nsrc, void* const* dst,
                                 int32_t ndst, size_t bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* tk_status_string(tk_status s);

/* TK_ENGRAM_ABI_VERSION of the built library. */
int32_t tk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TK_ENGRAM_H */
