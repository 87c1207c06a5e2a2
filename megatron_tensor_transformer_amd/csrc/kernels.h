// Internal launch interface between the C-ABI layer (api.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Operand storage order of a GEMM operand, seen from C = A·B with A (M×K) and
// B (K×N).
//   KMAJ : the K index is contiguous.  A: A[m*ld + k]; B: B[n*ld + k].
//   MNMAJ: the M (or N) index is contiguous.  A: A[k*ld + m]; B: B[k*ld + n].
enum OperandOrder { KMAJ = 0, MNMAJ = 1 };

// What the GEMM writes.
enum Epilogue {
  EPI_STORE = 0,      // C = acc (dtype of the path)
  EPI_STORE_F32 = 1,  // C = acc as fp32 (weight gradients)
  EPI_GELU_ZY = 2,    // C = acc (Z), C2 = GeLU(acc) (Y)
  EPI_GELU_GRAD = 3,  // C = acc ⊙ GeLU'(Zin) (D)
  EPI_BIAS_GELU_ZY = 4,  // z = acc + bias[col]: C = z (Z), C2 = GeLU(z) (Y)
  EPI_BIAS_STORE = 5,    // C = acc + bias[col] (dtype of the path)
  EPI_STORE_ROWSTATS = 6,  // C = acc (bf16), and per row and 64-column group of C as stored:
                           // (max, Σ exp(c − max)) into rstats (the cross-entropy's statistics)
  EPI_GELU_GRAD_DB = 7     // EPI_GELU_GRAD, and the column sums of C as stored over each
                           // 128-row chunk into colsum [batch][⌈M/128⌉][N] (the bias gradient's
                           // first stage)
};

struct GemmProblem {
  int M, N, K;
  int batch;
  const void* A;
  const void* B;
  void* C;
  void* C2;          // EPI_GELU_ZY: Y
  const void* Zin;   // EPI_GELU_GRAD: stored Z, same layout as C
  const void* bias;  // EPI_BIAS_GELU_ZY / EPI_BIAS_STORE: [N] per batch entry, path dtype
  int64_t sBias;     // its per-batch stride in elements
  float* rstats;     // EPI_STORE_ROWSTATS: [batch][M][⌈N/64⌉] pairs (max, sum) of floats
  float* colsum;     // EPI_GELU_GRAD_DB: [batch][⌈M/128⌉][N] column sums of 128-row chunks
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;  // per-batch strides in elements (0 = shared operand)
};

// bf16 inputs, fp32 accumulation (MFMA).  Returns a hipError_t.
hipError_t launch_gemm_bf16(const GemmProblem& p, int a_order, int b_order, int epi,
                            hipStream_t stream);
// Operand orders and epilogue of one GEMM problem.
struct GemmKind {
  int a_order, b_order, epi;
};

// Up to three independent problems in one launch (their tiles share one
// grid, so the machine stays full where each alone would leave part of it
// idle): a long group of nlong (≤ 2) problems of one kind, put first, and an
// optional short problem of another kind whose tiles fill in around them.
// Empty problems are skipped.  Supported: equal kinds, and a long group of
// (MNMAJ, MNMAJ, EPI_STORE_F32) with a short (KMAJ, KMAJ, EPI_STORE).
// With a workspace of at least gemm_bf16_split_bytes(...) bytes, problems
// that would leave the machine idle run K-split (fp32 partials in ws, then a
// fix-up kernel per split problem); with less (or none), nothing is split.
// The bf16 GEMM's tile and schedule policy (process-wide): TILE_AUTO picks
// 256×192 or 256×128 tiles or a K-split tail where a cost model of CU rounds
// favours them; TILE_256 uses none of them; TILE_192 and TILE_128 take
// 256×192 or 256×128 tiles wherever they are available (launches of one kind
// with the plain, GeLU, bias or GeLU' epilogue that run unsplit); TILE_STREAMK takes a K-split tail wherever it
// is available (launches of one problem, not fp32-output, whose 256×256 tiles
// fill at least one whole round of the CUs and at most half of another) and
// the workspace allows.
enum TilePolicy { TILE_AUTO = 0, TILE_256 = 1, TILE_192 = 2, TILE_STREAMK = 3, TILE_128 = 4 };
void set_gemm_tile_policy(int policy);
int gemm_tile_policy();

size_t gemm_bf16_split_bytes(const GemmProblem* longp, int nlong, const GemmKind& long_kind,
                             const GemmProblem* shortp, const GemmKind& short_kind);
hipError_t launch_gemm_bf16_group(const GemmProblem* longp, int nlong, const GemmKind& long_kind,
                                  const GemmProblem* shortp, const GemmKind& short_kind, void* ws,
                                  size_t ws_bytes, hipStream_t stream);
hipError_t launch_gemm_bf16_ws(const GemmProblem& p, int a_order, int b_order, int epi, void* ws, size_t ws_bytes,
                               hipStream_t stream);
// fp32 throughout.
hipError_t launch_gemm_f32(const GemmProblem& p, int a_order, int b_order, int epi,
                           hipStream_t stream);

// out = Σ_i partials[i]; dtypes: 0 = f32, 1 = bf16.
// out = Σ_i partials[i] (+ bias[col], bias NULL or [cols] of out_dt)
hipError_t launch_reduce_partials(int in_dt, int out_dt, int t, int64_t count,
                                  const void* partials, void* out, const void* bias, int64_t cols,
                                  hipStream_t stream);
// db[i][c] = Σ_r g[i][r][c] (fp32), via ws of t · bias_grad_chunks(rows) · cols floats
int64_t bias_grad_chunks(int64_t rows);
hipError_t launch_bias_grad(int dt, int t, int64_t rows, int64_t cols, const void* g, float* db, float* ws,
                            hipStream_t stream);
// the second stage alone: db[i][c] = Σ_chunk ws[i][chunk][c] in the fixed order
hipError_t launch_bias_grad_final(int t, int64_t rows, int64_t cols, float* db, const float* ws,
                                  hipStream_t stream);

struct SpProblem {
  int phase, dt, t;
  int64_t s, h, row0;
  float eps;
  uint32_t drop_threshold;
  float keep_scale;
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
  float* ws;
  const void* bias;  // DROPRES_FWD: NULL or [h] of dt, added to Σ_i P_i before the dropout
};

// LN backward's per-block column partials: row blocks of the grid, and the
// floats of the SP workspace (the partials, plus two row means per row when
// h > 4096)
int64_t sp_ln_bwd_row_blocks(int64_t s, int64_t h);
int64_t sp_workspace_floats(int64_t s, int64_t h);

// Attention core of T resident shards (layouts in attention.hip).
struct AttnProblem {
  int dt, T, s, b, nh, dh;
  bool causal;
  const uint32_t* mask;  // packed general mask (launch_attn_pack_mask), or null
  const void* qkv;   // [T][s·b][nh·3·dh]
  void* o;           // [T][s·b][nh·dh]
  float* lse;        // [T][b][nh][s]
  const void* dout;  // backward: upstream gradient of o, layout of o
  void* dqkv;        // backward: layout of qkv
  float* delta;      // backward workspace [T][b][nh][s]
};
hipError_t launch_attn_fwd(const AttnProblem& p, hipStream_t stream);
// Byte mask [b][s][s] -> the packed form the attention kernels read:
// 2·b·s·⌈s/32⌉ words (rows part, then columns part).
hipError_t launch_attn_pack_mask(int b, int s, const uint8_t* mask, uint32_t* packed, hipStream_t stream);

// Vocabulary-parallel cross-entropy of T resident shards (vocab_ce.hip).
struct VocabProblem {
  int dt, T;
  int64_t n, vi, start0;  // tokens, vocabulary entries per shard, first entry of shard 0
  const void* logits;     // [T][n][vi]
  const int* target;      // [n], global vocabulary ids
  float* stats;           // workspace [T][n][⌈vi/64⌉] pairs (max, Σ exp(x − max)) per 64-column group
  bool stats_done;        // the logit GEMM's epilogue has written stats (bf16 path)
  float* loss;            // [n]
  float* rmax;            // [n] row max over all shards
  float* rsum;            // [n] Σ exp(x − rmax) over all shards
  const float* g;         // backward: [n] upstream gradient of each loss
  void* dlogits;          // backward: [T][n][vi]
};
hipError_t launch_vocab_ce_fwd(const VocabProblem& p, hipStream_t stream);
hipError_t launch_vocab_ce_bwd(const VocabProblem& p, hipStream_t stream);
hipError_t launch_attn_bwd(const AttnProblem& p, hipStream_t stream);
hipError_t launch_sp(const SpProblem& p, hipStream_t stream);

}  // namespace tpmlp
