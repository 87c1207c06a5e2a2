/*
 * tpmlp.h -- C ABI of the tensor-parallel MLP shard library for AMD MI355X
 * (gfx950).  Every entry point enqueues HIP kernels on the caller's stream and
 * returns; nothing here allocates or keeps a pointer after returning.  The
 * only host state is the per-thread code of the last failed launch
 * (tpmlp_last_hip_error), the process-wide GEMM tile policy
 * (tpmlp_set_gemm_tile_policy, an atomic integer) and, once
 * tpmlp_bias_grad_noalloc has run on a device, that device's address of the
 * library's fixed scratch array (looked up once, under a lock).  The library
 * is thread-safe.
 *
 * Sources (page title, section):
 *   [TUT]   "024｜Megatron-LM：按矩阵结构切分 Transformer，减少模型并行通信",
 *           §二 "前向少通信，反向为何仍要一次归约？" -- the shard forward
 *           Z_i = X·A_i, Y_i = φ(Z_i), O = Σ_i Y_i·B_i and the shard backward
 *           D_i = (G·B_iᵀ)⊙φ'(Z_i), ∂ℓ/∂A_i = Xᵀ·D_i, ∂ℓ/∂B_i = Y_iᵀ·G,
 *           ∂ℓ/∂X = Σ_i D_i·A_iᵀ.
 *   [SENSE] SenseParrots 模型并行 (xujun.org), §2.1 Eq.(1)/(2): column split
 *           of the first weight, row split of the second; splits are even.
 *   [SP]    "Megatron-SP 机制", sections on the f/g operator table, the layer
 *           placement diagram and the RNG-domain table: LayerNorm, dropout and
 *           residual run on the rank's s/t rows; AllGather before fc1,
 *           ReduceScatter after fc2.
 *   [TRAIN] "Megatron 训练" (lovelonelytime), LayerNorm and Dropout sections;
 *           ColumnParallelLinear / RowParallelLinear (where each layer's bias
 *           lives) and the custom autograd matmul (its gradient).
 *   [EFF]   notes on "Efficient Large-Scale Language Model Training on GPU
 *           Clusters Using Megatron-LM" (unpurerationalist.github.io), §4.2:
 *           bias + GeLU and bias + dropout + add fused into single kernels;
 *           the sequence-first [s, b, a, h] layout and the fused scale + mask
 *           + softmax with an implicit causal mask.
 * The attention entry points also follow [SENSE] §2.1.1 (the multi-head
 * attention paragraph and module: heads split over shards, qkv
 * column-parallel without gather, proj row-parallel with a split input) and
 * [TRAIN] "Attention 层" (S = QKᵀ/√d, A = softmax(S), its gradient).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers to row-major, contiguous tensors.  Shapes
 *     are given in elements.  A tensor of dtype bf16 is IEEE bfloat16; f32 is
 *     IEEE binary32.
 *   - Shards: t_local shards are resident together and processed by the same
 *     launch; per-shard tensors are stacked along a leading shard axis.
 *   - Outputs are overwritten, never accumulated into.
 *   - Validation happens before any launch.  A negative status means nothing
 *     was enqueued, except TPMLP_ERR_HIP, which reports a failed launch
 *     (earlier kernels of the same call may have been enqueued).
 *   - The caller owns every buffer and keeps it alive until the stream work
 *     completes.  Inputs and outputs must not overlap.
 *   - A call issues no allocation, memset, copy or synchronisation, only
 *     kernel launches, so a sequence of calls may be captured into a HIP
 *     graph on the caller's stream and replayed (replays read the buffers'
 *     contents at replay time).
 *   - bf16 operands need 16-byte aligned base pointers and row lengths that
 *     are multiples of 8 elements (d % 8 == 0, m_i % 8 == 0); so do the fp32
 *     weight gradients the bf16 path writes (dA, dB, dW_qkv, dW_proj, dW:
 *     16-byte aligned, written with 16-byte stores).  On the f32 path the
 *     GEMM operands and outputs need 4-byte alignment only; tpmlp_ln_sp has
 *     its own rules (below).  Each per-shard operand must be smaller than
 *     2^31 bytes.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPMLP_ABI_VERSION 9

typedef enum { TPMLP_F32 = 0, TPMLP_BF16 = 1 } tpmlp_dtype;

enum {
  TPMLP_OK = 0,
  TPMLP_ERR_NULLPTR = -1,   /* a required pointer is NULL                        */
  TPMLP_ERR_SHAPE = -2,     /* negative/zero size, shard split not even, t < 2 for SP */
  TPMLP_ERR_DTYPE = -3,     /* unknown dtype or unsupported dtype combination    */
  TPMLP_ERR_ALIGN = -4,     /* bf16 base pointer not 16-B aligned or row length % 8 */
  TPMLP_ERR_HIP = -5,       /* a kernel launch failed (tpmlp_last_hip_error)     */
  TPMLP_ERR_WORKSPACE = -6, /* workspace missing or smaller than required        */
  TPMLP_ERR_ARG = -7,       /* other invalid argument (phase, probability, eps)  */
  TPMLP_ERR_SCRATCH = -8    /* more scratch needed than an allocation-free entry
                               point's fixed array holds                         */
};

/*
 * tpmlp_fwd -- forward of t_local MLP shards ([TUT] §二; [SENSE] Eq.(1)/(2)).
 *
 *   Z_i = X·A_i          [n, m_i]   (stored: the backward needs it)
 *   Y_i = GeLU(Z_i)      [n, m_i]   the erf GeLU z·Φ(z), evaluated on the
 *                                   fp32 accumulator before Z_i is rounded.
 *                                   f32 path: erff from the device library.
 *                                   bf16 path: a clamped odd polynomial of
 *                                   degree 9 in z² for Φ on |z| <= 4.5 (Φ
 *                                   exactly 0 / 1 beyond), |GeLU error| <=
 *                                   7e-5 over all z, far below bf16's 2^-9
 *                                   relative resolution
 *   P_i = Y_i·B_i        [n, d]     row-parallel partial output; O = Σ_i P_i
 *                                   is formed by tpmlp_reduce_partials
 *
 *   dt      TPMLP_BF16 (fp32 accumulation) or TPMLP_F32 (fp32 throughout)
 *   n       tokens (b·s), n >= 0; n == 0 enqueues nothing
 *   d       model width, d >= 1
 *   m_i     hidden columns per shard (m / t), m_i >= 1
 *   t_local shards processed by this call, >= 1
 *   X [n, d]; A [t_local, d, m_i] (shard i = column block i of the full
 *   first weight); B [t_local, m_i, d] (shard i = row block i of the full
 *   second weight); Z, Y [t_local, n, m_i]; P [t_local, n, d]; all of dt.
 *   ws / ws_bytes: workspace of at least tpmlp_fwd_workspace_bytes(dt, n, d,
 *   m_i, t_local) bytes, 16-byte aligned (may be NULL when that is 0; less
 *   is TPMLP_ERR_WORKSPACE).  It is non-zero only for bf16 shapes whose
 *   products have too few 256×256 output tiles to fill the GPU: those run
 *   K-split (each K slice's fp32 partial tile in ws, then a fix-up kernel
 *   adds the slices in a fixed order and applies the GeLU or plain
 *   epilogue).  The split depends only on the sizes, so results are
 *   bit-reproducible; they differ from an unsplit product only by the fp32
 *   summation order.
 */
size_t tpmlp_fwd_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local);
int tpmlp_fwd(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
              const void* X, const void* A, const void* B, void* Z, void* Y, void* P, void* ws, size_t ws_bytes);

/*
 * tpmlp_fwd_bias -- tpmlp_fwd with the first layer's bias.  The column-
 * parallel layer's bias is split like its output columns, so shard i owns
 * slice i and adds it before the activation ([TRAIN] ColumnParallelLinear);
 * the add and the GeLU run in the GEMM's epilogue ([EFF] §4.2):
 *
 *   Z_i = X·A_i + 1·b1_iᵀ   (added to the fp32 accumulator, then rounded)
 *   Y_i = GeLU(Z_i),  P_i = Y_i·B_i
 *
 *   b1 [t_local, m_i] of dt (row i = slice i of the full bias), not NULL.
 *   Everything else, errors included, as for tpmlp_fwd; the workspace is
 *   tpmlp_fwd_bias_workspace_bytes(...) bytes.  The backward is tpmlp_bwd
 *   unchanged (Z_i already holds the bias), plus tpmlp_bias_grad.
 */
size_t tpmlp_fwd_bias_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local);
int tpmlp_fwd_bias(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
                   const void* X, const void* A, const void* B, const void* b1, void* Z, void* Y, void* P, void* ws,
                   size_t ws_bytes);

/*
 * tpmlp_bwd -- backward of t_local MLP shards ([TUT] §二).
 *
 *   D_i   = (G·B_iᵀ) ⊙ GeLU'(Z_i)   [n, m_i]  dt; GeLU' = Φ(z) + z·ϕ(z) is
 *                                            evaluated on the stored Z_i
 *                                            (f32 path: erff / expf; bf16
 *                                            path: the same kind of clamped
 *                                            polynomial as the forward,
 *                                            |GeLU' error| <= 1.5e-4)
 *   dA_i  = Xᵀ·D_i                  [d, m_i]  fp32
 *   dB_i  = Y_iᵀ·G                  [m_i, d]  fp32
 *   dX_i  = D_i·A_iᵀ                [n, d]    dt, partial input gradient;
 *                                            dX = Σ_i dX_i is formed by
 *                                            tpmlp_reduce_partials
 *
 *   Inputs X, A, B as for tpmlp_fwd; Z, Y from tpmlp_fwd; G [n, d] the
 *   upstream gradient ∂ℓ/∂O.  With n == 0, dA and dB are set to zero.
 *   dA and dB: 16-byte aligned on the bf16 path, 4-byte on the f32 path.
 *   ws / ws_bytes: workspace, at least tpmlp_bwd_workspace_bytes(...) bytes,
 *   16-byte aligned (may be NULL when that is 0; less is
 *   TPMLP_ERR_WORKSPACE): as for tpmlp_fwd, products that would leave the
 *   GPU idle (few output tiles, long K) run K-split there.
 */
size_t tpmlp_bwd_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local);
int tpmlp_bwd(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
              const void* X, const void* A, const void* B, const void* Z, const void* Y,
              const void* G, void* D, float* dA, float* dB, void* dXp, void* ws, size_t ws_bytes);

/*
 * tpmlp_bwd_bias -- tpmlp_bwd of the biased layer (tpmlp_fwd_bias), with the
 * two bias gradients ([TRAIN] custom autograd matmul: a bias broadcast over
 * the rows gets the upstream gradient summed over the rows):
 *
 *   db1_i = Σ_rows D_i   [t_local, m_i] fp32 (the column-parallel bias,
 *                        split like A's columns)
 *   db2   = Σ_rows G     [d] fp32 (the row-parallel bias, added once)
 *
 * On the bf16 path the column sums of D are taken in the dgrad-1 GEMM's
 * epilogue, of the values as stored (bf16), per 128-row chunk ([EFF] §4.2:
 * the bias work fused into the GEMM instead of a pass over D); the chunk
 * sums are then added in chunk order.  db2 is a two-stage column sum of G
 * as in tpmlp_bias_grad.  Both orders are fixed, so results are
 * bit-reproducible; db1 differs from tpmlp_bias_grad's over the stored D only
 * by the fp32 summation order.
 *
 *   Everything else as for tpmlp_bwd; db1, db2 not NULL, 4-byte aligned;
 *   t_local <= 65535.  With n == 0, dA, dB, db1 and db2 are set to zero.
 *   ws / ws_bytes: at least tpmlp_bwd_bias_workspace_bytes(...) bytes,
 *   16-byte aligned (the chunk sums of D and G, plus tpmlp_bwd's split
 *   partials of the weight-gradient launch; dgrad-1 is never split here).
 */
size_t tpmlp_bwd_bias_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local);
int tpmlp_bwd_bias(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
                   const void* X, const void* A, const void* B, const void* Z, const void* Y, const void* G, void* D,
                   float* dA, float* dB, void* dXp, float* db1, float* db2, void* ws, size_t ws_bytes);

/*
 * tpmlp_reduce_partials -- out = Σ_{i=0}^{t-1} partials[i]  (the one-GPU
 * stand-in for the all-reduce after the row-parallel GEMM and for the
 * all-reduce of the column-parallel input gradient: [TRAIN] RowParallelLinear
 * forward / ColumnParallelLinear backward; a sum, never a mean, [TUT] §三).
 * Accumulation is fp32 in the fixed order i = 0, 1, ..., t-1, so results are
 * bit-reproducible.
 *
 *   in_dt, out_dt  TPMLP_BF16 or TPMLP_F32 each
 *   partials [t, rows, cols] of in_dt; out [rows, cols] of out_dt
 *   t >= 1, rows >= 0, cols >= 1
 */
int tpmlp_reduce_partials(hipStream_t stream, int in_dt, int out_dt, int32_t t, int64_t rows,
                          int64_t cols, const void* partials, void* out);

/*
 * tpmlp_reduce_partials_bias -- out = Σ_i partials[i] + 1·biasᵀ.  The
 * row-parallel layer's bias is not split: it is added once, after the
 * all-reduce ([TRAIN] RowParallelLinear).  The fp32 shard-order sum is formed
 * as in tpmlp_reduce_partials, then bias[c] is added in fp32 and the result
 * rounded once to out_dt.
 *
 *   bias [cols] of out_dt, not NULL; other arguments as for
 *   tpmlp_reduce_partials.
 */
int tpmlp_reduce_partials_bias(hipStream_t stream, int in_dt, int out_dt, int32_t t, int64_t rows,
                               int64_t cols, const void* partials, const void* bias, void* out);

/*
 * tpmlp_bias_grad -- db[i] = Σ_r g[i][r]: the gradient of a bias broadcast
 * over rows is the upstream gradient summed over the rows ([TRAIN] custom
 * autograd matmul).  For the MLP: db1_i = Σ_rows D_i (g = D, t = t_local,
 * cols = m_i) and db2 = Σ_rows G (g = G, t = 1, cols = d; under sequence
 * parallelism g = dS).
 *
 *   dt    dtype of g (TPMLP_BF16 or TPMLP_F32)
 *   g     [t, rows, cols]; db [t, cols] fp32
 *   The sum is fp32 in a fixed order, so results are bit-reproducible:
 *   column partials of 128-row chunks (rows in increasing order within each
 *   of 8 interleaved row phases, the phases added in order), then the chunk
 *   partials in 8 consecutive ranges (each in increasing order, the ranges
 *   added in order).  rows == 0 sets db to
 *   zero and needs no g or workspace.
 *   ws / ws_bytes: at least tpmlp_bias_grad_workspace_bytes(t, rows, cols)
 *   bytes, 4-byte aligned.
 *   Limits: t <= 65535; ceil(cols/32)·ceil(rows/128) < 2^31;
 *   ceil(t·cols/32) < 2^31.
 */
size_t tpmlp_bias_grad_workspace_bytes(int32_t t, int64_t rows, int64_t cols);
int tpmlp_bias_grad(hipStream_t stream, int dt, int32_t t, int64_t rows, int64_t cols, const void* g,
                    float* db, void* ws, size_t ws_bytes);

/*
 * tpmlp_bias_grad_noalloc -- tpmlp_bias_grad without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (minus ws / ws_bytes), kernels, fixed
 * summation order and results, bit for bit, as tpmlp_bias_grad.
 *
 * The chunk partials go to a fixed device array of the library,
 * TPMLP_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, which each GPU the library
 * runs on holds until the process ends; its address is looked up on the
 * first call on a device.  A call whose tpmlp_bias_grad_workspace_bytes(t,
 * rows, cols) exceeds it returns TPMLP_ERR_SCRATCH with nothing enqueued
 * (the 8.3B-shaped layer's db1, t = 8, rows = 8192, cols = 1536, needs
 * 3 MiB).  The array is shared by every call on that GPU and keeps the last
 * call's contents (nothing in it needs clearing: each call writes every
 * partial it reads); calls that overlap on one GPU (other streams, other
 * threads) race on it and must be serialised by the caller.  A failed
 * address lookup returns TPMLP_ERR_HIP.
 */
#define TPMLP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int tpmlp_bias_grad_noalloc(hipStream_t stream, int dt, int32_t t, int64_t rows, int64_t cols, const void* g,
                            float* db);

/*
 * tpmlp_ln_sp -- the sequence-parallel region around one MLP block
 * ([SP] placement diagram; [TRAIN] LayerNorm and Dropout sections):
 *     out = x + dropout_p( Σ_i P_i ),   the MLP input being LN(x)
 * With a bias (a->bias not NULL; [TRAIN] RowParallelLinear: the unsplit bias
 * of the second layer is added after the reduction) the forward is
 *     out = x + dropout_p( Σ_i P_i + b2 )
 * with the bias add, dropout and residual add in one kernel ([EFF] §4.2).
 * The t sequence shards of s/t rows each are all resident (s rows in total);
 * the AllGather before fc1 is the row-block layout of ln_out itself, and the
 * ReduceScatter after fc2 is a sum over the t partials whose row blocks are
 * the shards.  The dropout keep-mask is regenerated, never stored: element
 * (r, c) with global index e = (row0 + r)·h + c is dropped iff word (e mod 4)
 * of Philox-4x32-10(counter = (e div 4) as two 32-bit words + two zero words,
 * key = seed as two 32-bit words) is below floor(p·2^32); survivors are scaled
 * by 1/(1-p).  Every sequence shard therefore draws its own mask.
 *
 * Phases (a->phase):
 *   TPMLP_SP_LN_FWD      x, gamma, beta -> ln_out [s,h] (dt), mean, rstd [s] (f32)
 *   TPMLP_SP_DROPRES_FWD partials [t,s,h] (the MLP's P_i), x, bias [h] or
 *                        NULL -> out [s,h]
 *   TPMLP_SP_DROPRES_BWD g_out [s,h] -> dS [s,h] = g_out⊙mask/(1-p)
 *                        (the MLP's upstream gradient G)
 *   TPMLP_SP_LN_BWD      dU_partials [t,s,h] (the MLP's dX_i), g_out, x,
 *                        gamma, mean, rstd -> dx = g_out + LN'(Σ_i dU_i) [s,h],
 *                        dgamma, dbeta [h] (f32, summed over all s rows in a
 *                        fixed order; needs ws)
 * LayerNorm: biased variance over h, eps inside the square root, statistics
 * in fp32.  Requirements (checked; SHAPE, ALIGN or ARG otherwise):
 *   - t >= 2 (sequence parallelism needs tensor parallelism, [SP] 工程约束),
 *     s >= 0, s % t == 0, row0 >= 0;
 *   - h >= 8 and h % 8 == 0 for both dtypes (the kernels move 8-element
 *     chunks); any such width: rows wider than 4096 take a slower
 *     multi-pass path (the row is re-read from the cache per pass, and LN
 *     backward forms its two row means in a pass of their own);
 *   - every tensor pointer 16-byte aligned for both dtypes (f32 included);
 *     mean, rstd, dgamma, dbeta 4-byte aligned;
 *   - s·h and t·s·h elements of dt each smaller than 2^31 bytes;
 *   - 0 <= p < 1, eps > 0.
 * s == 0 enqueues nothing.  LN_BWD's workspace: tpmlp_sp_workspace_bytes(s,
 * h) bytes, 4-byte aligned (per-block column partials of dγ/dβ, plus two row
 * means per row when h > 4096).
 */
typedef enum {
  TPMLP_SP_LN_FWD = 0,
  TPMLP_SP_DROPRES_FWD = 1,
  TPMLP_SP_DROPRES_BWD = 2,
  TPMLP_SP_LN_BWD = 3
} tpmlp_sp_phase;

typedef struct {
  int32_t phase;            /* tpmlp_sp_phase                                   */
  int32_t dt;               /* dtype of x, gamma, beta, ln_out, partials, out,
                               g_out, dS, dU_partials, dx                       */
  int32_t t;                /* SP degree = TP degree = number of partials       */
  int32_t reserved;
  int64_t s;                /* rows on this GPU (all t shards)                  */
  int64_t h;                /* hidden width                                     */
  int64_t row0;             /* global index of row 0 (mask counter offset)      */
  float eps;
  float p_drop;
  uint64_t seed;
  const void* x;
  const void* gamma;
  const void* beta;
  void* ln_out;
  float* mean;
  float* rstd;
  const void* partials;
  void* out;
  const void* g_out;
  void* dS;
  const void* dU_partials;
  void* dx;
  float* dgamma;
  float* dbeta;
  void* ws;
  size_t ws_bytes;
  const void* bias;         /* DROPRES_FWD: [h] of dt, or NULL (no bias); ignored
                               by the other phases                              */
} tpmlp_sp_args;

size_t tpmlp_sp_workspace_bytes(int64_t s, int64_t h);
int tpmlp_ln_sp(hipStream_t stream, const tpmlp_sp_args* a);

/*
 * Self-attention shard ([SENSE] §2.1.1; [TRAIN] Attention 层; [EFF] §4.2).
 * Shard i of the layer owns heads_local consecutive heads of width head_dim
 * (w = heads_local·head_dim): the column block W_qkv,i [d, 3w] of the QKV
 * weight, whose columns go head by head as (q | k | v, head_dim), and the
 * row block W_proj,i [w, d] of the output projection.  Tokens are the rows of
 * X [n, d], n = s·b, in sequence-first order: row s_idx·b + b_idx.
 *
 *   QKV_i = X·W_qkv,i                       [n, 3w]
 *   per batch entry and head: S = q·kᵀ/√head_dim, with causal != 0 the
 *   entries of key positions after the query position are −∞, and with a
 *   general mask the entries it hides are −∞ as well; A = softmax of each
 *   row of S; o = A·v (a row that sees no key: o = 0, lse = −∞, and it
 *   passes no gradient)
 *   O_i  = the heads' o side by side        [n, w]
 *   P_i  = O_i·W_proj,i                     [n, d]  row-parallel partial;
 *                                                   Σ_i P_i via
 *                                                   tpmlp_reduce_partials
 *   lse_i[b][h][s] = ln Σ_j exp(S_ij)       fp32, kept for the backward
 * Backward, G = ∂ℓ/∂Σ_i P_i [n, d]:
 *   dO_i = G·W_proj,iᵀ;  dW_proj,i = O_iᵀ·G (fp32)
 *   per head: dv = Aᵀ·do;  dS = A ⊙ (do·vᵀ − δ), δ = rowsum(do ⊙ o);
 *             dq = dS·k/√head_dim;  dk = dSᵀ·q/√head_dim  -> dQKV_i [n, 3w]
 *   dW_qkv,i = Xᵀ·dQKV_i (fp32);  dX_i = dQKV_i·W_qkv,iᵀ   partial, summed by
 *                                                   tpmlp_reduce_partials
 * The attention dropout is not applied (the module on [SENSE] defaults it to
 * 0).
 *
 * Biases ([TRAIN] ColumnParallelLinear / RowParallelLinear, as for the MLP):
 * tpmlp_attn_fwd_bias adds the QKV column bias bqkv [t_local, 3w] (shard i's
 * slice of b_qkv, path dtype, same alignment as the weights; NULL is NULLPTR)
 * in the QKV GEMM's epilogue: QKV_i = X·W_qkv,i + bqkv_i.  The projection's
 * bias is added once after the sum (tpmlp_reduce_partials_bias).  Their
 * gradients are column sums (tpmlp_bias_grad): db_qkv,i = Σ_rows dQKV_i,
 * db_proj = Σ_rows G.  The backward is unchanged.
 *
 *   dt          TPMLP_BF16 (flash-attention kernels on the matrix cores, fp32
 *               softmax statistics) or TPMLP_F32 (fp32 throughout)
 *   s, b        sequence length (>= 0; 0 enqueues nothing) and batch (>= 1)
 *   heads_local heads per shard (>= 1); head_dim 64 or 128
 *   t_local     shards processed by this call (>= 1), stacked on a leading
 *               axis of every per-shard tensor
 *   causal      0 (no mask) or 1 (causal)
 *   mask        null (none) or a general mask packed by tpmlp_attn_pack_mask
 *               (4-byte aligned): it hides key position j from query
 *               position i of batch entry β for every head and shard — the
 *               general mask of [EFF] §4.2's fused softmax (BERT's padding
 *               mask is one); combined with causal when both are given.
 * Layouts: X [n, d]; W_qkv [t_local, d, 3w]; W_proj [t_local, w, d];
 *   QKV, dQKV [t_local, n, 3w]; O, dO [t_local, n, w]; lse [t_local, b,
 *   heads_local, s] fp32; P, dXp [t_local, n, d]; dW_qkv [t_local, d, 3w]
 *   and dW_proj [t_local, w, d] fp32.
 * Limits: one shard's QKV smaller than 2^31 bytes; t_local·b·heads_local·s
 *   < 2^31; with a mask, 4·s·⌈s/32⌉ < 2^31; bf16 needs d % 8 == 0 and
 *   16-byte aligned bases.
 * Workspace of the backward: tpmlp_attn_bwd_workspace_bytes(...) bytes (the
 * δ rows), 4-byte aligned.
 * No atomics: every output is summed in a fixed order that depends only on
 * the sizes (which kernels run, and how work is dealt to workgroups, too), so
 * results are bit-reproducible.
 *
 * tpmlp_attn_core_fwd / _bwd run the attention core alone on a given QKV
 * (and O, lse, dO): QKV -> O, lse and (QKV, O, lse, dO) -> dQKV.
 *
 * General mask, packed once per batch and read by every layer and both
 * passes: tpmlp_attn_pack_mask turns a byte mask [b][s][s] (mask[β][i][j] !=
 * 0 hides key j from query i; caller-owned device memory, any alignment) into
 * tpmlp_attn_mask_words(b, s) 32-bit words (W = ⌈s/32⌉; part 0 [b][s][W] by
 * query row: bit j of word w = key 32w + j hidden; part 1 [b][s][W] by key
 * column: bit i of word w = query 32w + i hidden; positions past s set).
 * tpmlp_attn_mask_words returns 0 for b < 1 or s < 1.  Errors: SHAPE (b < 1,
 * s < 0, 4·s·W >= 2^31), NULLPTR, ALIGN (packed not 4-byte aligned); s = 0
 * enqueues nothing.
 */
size_t tpmlp_attn_mask_words(int64_t b, int64_t s);
int tpmlp_attn_pack_mask(hipStream_t stream, int64_t b, int64_t s, const uint8_t* mask, uint32_t* packed);
int tpmlp_attn_fwd(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                   int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                   const void* Wqkv, const void* Wproj, void* QKV, void* O, float* lse, void* P);
int tpmlp_attn_fwd_bias(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                        int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                        const void* Wqkv, const void* Wproj, const void* bqkv, void* QKV, void* O, float* lse,
                        void* P);
size_t tpmlp_attn_bwd_workspace_bytes(int32_t t_local, int64_t s, int64_t b, int32_t heads_local);
int tpmlp_attn_bwd(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                   int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                   const void* Wqkv, const void* Wproj, const void* QKV, const void* O, const float* lse,
                   const void* G, void* dO, void* dQKV, float* dWqkv, float* dWproj, void* dXp, void* ws,
                   size_t ws_bytes);
int tpmlp_attn_core_fwd(hipStream_t stream, int dt, int32_t t_local, int64_t s, int64_t b, int32_t heads_local,
                        int32_t head_dim, int causal, const uint32_t* mask, const void* qkv, void* o, float* lse);
int tpmlp_attn_core_bwd(hipStream_t stream, int dt, int32_t t_local, int64_t s, int64_t b, int32_t heads_local,
                        int32_t head_dim, int causal, const uint32_t* mask, const void* qkv, const void* o,
                        const float* lse, const void* d_o, void* dqkv, void* ws, size_t ws_bytes);

/*
 * Vocabulary-parallel logit layer and cross-entropy ([SENSE] §2.2.2, Eq. (3)
 * and (4); the logit layer's FLOPs per [EFF]'s appendix).  Shard i owns
 * vocabulary entries [vocab_start + i·v_i, vocab_start + (i+1)·v_i): rows
 * W_i [v_i, h] of the embedding table.
 *
 * tpmlp_vocab_ce_fwd:
 *   logits_i = X·W_iᵀ                              [n, v_i]  dt
 *   per shard and token: m_i = max, s_i = Σ exp(x − m_i), τ_i = target logit
 *   if the target is the shard's entry, else 0; combined by a max and two
 *   sums (the three small all-reduces of the page):
 *   row_max = max_i m_i, row_sum = Σ_i s_i·exp(m_i − row_max),
 *   loss = ln(row_sum) + row_max − Σ_i τ_i          [n] fp32 each
 *   The statistics are those of the logits as stored; they are taken per 64
 *   columns (on the bf16 path in the logit GEMM's epilogue) and combined in a
 *   fixed order.
 * tpmlp_vocab_ce_bwd, g [n] fp32 = ∂ℓ/∂loss (1/n for the mean loss):
 *   dlogits_i = g·(exp(logits_i − row_max)/row_sum − onehot(target))   dt
 *   dW_i = dlogits_iᵀ·X  [v_i, h] fp32;  dX_i = dlogits_i·W_i [n, h] dt
 *   (partial: dX = Σ_i dX_i by tpmlp_reduce_partials)
 *
 *   X [n, h]; W [t_local, v_i, h]; targets [n] int32 global vocabulary ids;
 *   logits, dlogits [t_local, n, v_i]; dW [t_local, v_i, h]; dXp [t_local,
 *   n, h].  Exponentials and sums in fp32.  A target outside the resident
 *   shards contributes no target logit (its owner is another rank).
 *   bf16 needs h % 8 == 0 and v_i % 8 == 0 (as d and m_i of tpmlp_fwd).
 *   Workspace of the forward: tpmlp_vocab_ce_workspace_bytes(t_local, n,
 *   v_i) bytes (a pair of floats per shard, token and 64 columns), 8-byte
 *   aligned.
 */
size_t tpmlp_vocab_ce_workspace_bytes(int32_t t_local, int64_t n, int64_t v_i);
int tpmlp_vocab_ce_fwd(hipStream_t stream, int dt, int64_t n, int64_t h, int64_t v_i, int32_t t_local,
                       int64_t vocab_start, const void* X, const void* W, const int32_t* targets, void* logits,
                       float* loss, float* row_max, float* row_sum, void* ws, size_t ws_bytes);
int tpmlp_vocab_ce_bwd(hipStream_t stream, int dt, int64_t n, int64_t h, int64_t v_i, int32_t t_local,
                       int64_t vocab_start, const void* X, const void* W, const int32_t* targets,
                       const void* logits, const float* row_max, const float* row_sum, const float* g,
                       void* dlogits, float* dW, void* dXp);

/*
 * Tile width and schedule of the bf16 GEMMs, a tuning and testing knob
 * (process-wide; calls already enqueued are not affected).
 *   TPMLP_GEMM_TILE_AUTO (default): per launch, from its shapes, 256×192 or
 *     256×128 output tiles instead of 256×256 where they fill the GPU's 256
 *     compute units in fewer rounds of tiles (one-kind launches with the
 *     plain, GeLU, GeLU' or bias epilogue that run without a K split; e.g.
 *     one shard of the 8.3B-shaped layer, n = 8192, m_i = 1536: 256 tiles of
 *     256×192 instead of 192; the single-shard layer's 2048×4096 products:
 *     256 tiles of 256×128 instead of 128),
 *     or a K-split tail where a launch of one problem fills whole rounds and
 *     at most half of another (e.g. the GPT-1T-shaped shard's P = Y·B_i: 800
 *     tiles, 3 rounds and 32 more): each leftover tile runs as q equal K
 *     pieces (q·tiles ≤ 256) of fp32 partials in the workspace, added by a
 *     fix-up kernel in K order.
 *   TPMLP_GEMM_TILE_256: 256×256 tiles, no K-split tail.
 *   TPMLP_GEMM_TILE_192, TPMLP_GEMM_TILE_128: 256×192 or 256×128 tiles
 *     wherever they are available.
 *   TPMLP_GEMM_STREAMK: a K-split tail wherever it is available (the
 *     workspace queries then ask for its partial tiles, 256 KiB each).
 * Narrow tiles give the same results as 256×256 bit for bit (each output
 * element's K sum runs in the same order); a K-split tail adds the tail
 * tiles' K sums in q fp32 pieces (a different rounding, the same on every
 * run).  Returns TPMLP_OK, or TPMLP_ERR_ARG for another value.
 */
#define TPMLP_GEMM_TILE_AUTO 0
#define TPMLP_GEMM_TILE_256 1
#define TPMLP_GEMM_TILE_192 2
#define TPMLP_GEMM_STREAMK 3
#define TPMLP_GEMM_TILE_128 4
int tpmlp_set_gemm_tile_policy(int policy);
int tpmlp_gemm_tile_policy(void);

/* Status text for a return code; never NULL. */
const char* tpmlp_status_string(int status);
/* The hipError_t of the most recent TPMLP_ERR_HIP on the calling thread. */
int tpmlp_last_hip_error(void);
int tpmlp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */
