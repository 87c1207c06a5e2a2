// C ABI of the tensor-parallel MLP shard library: argument validation and the
// mapping of each step onto the kernels.  Validation never touches the GPU, so
// every error status is returned with nothing enqueued.
#include <math.h>
#include <initializer_list>
#include <mutex>
#include <stdint.h>

#include "../../include/tpmlp.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxOperandBytes = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

int elem_size(int dt) { return dt == TPMLP_BF16 ? 2 : 4; }
bool valid_dt(int dt) { return dt == TPMLP_BF16 || dt == TPMLP_F32; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool fits(int64_t rows, int64_t cols, int es) {
  if (rows < 0 || cols < 0) return false;
  if (cols != 0 && rows > kMaxOperandBytes / cols) return false;
  return rows * cols * es <= kMaxOperandBytes;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TPMLP_OK;
  g_last_hip_error = static_cast<int>(e);
  return TPMLP_ERR_HIP;
}

// Shared checks of tpmlp_fwd / tpmlp_bwd dimensions.
int check_mlp_dims(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  if (!valid_dt(dt)) return TPMLP_ERR_DTYPE;
  if (n < 0 || d < 1 || m_i < 1 || t_local < 1) return TPMLP_ERR_SHAPE;
  if (n > kMaxDim || d > kMaxDim || m_i > kMaxDim) return TPMLP_ERR_SHAPE;
  const int es = elem_size(dt);
  if (!fits(n, d, es) || !fits(d, m_i, es) || !fits(n, m_i, es) || !fits(d, m_i, 4))
    return TPMLP_ERR_SHAPE;
  if (dt == TPMLP_BF16 && (d % 8 != 0 || m_i % 8 != 0)) return TPMLP_ERR_ALIGN;
  return TPMLP_OK;
}

// fp32 weight gradients: the bf16 path's GEMM epilogue writes them with 16-B
// vector stores (4 consecutive columns; rows are multiples of 8 columns)
uintptr_t wgrad_align(int dt) { return dt == TPMLP_BF16 ? 16 : 4; }

int check_ptrs(int dt, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return TPMLP_ERR_NULLPTR;
  const uintptr_t a = dt == TPMLP_BF16 ? 16 : 4;
  for (const void* p : ps)
    if (!aligned(p, a)) return TPMLP_ERR_ALIGN;
  return TPMLP_OK;
}

hipError_t gemm(int dt, const tpmlp::GemmProblem& p, int ao, int bo, int epi, hipStream_t s) {
  return dt == TPMLP_BF16 ? tpmlp::launch_gemm_bf16(p, ao, bo, epi, s)
                          : tpmlp::launch_gemm_f32(p, ao, bo, epi, s);
}

// The forward's two products (pointers may be null for a size query).
void fwd_problems(int64_t n, int64_t d, int64_t m_i, int32_t t_local, const void* X, const void* A, const void* B,
                  const void* b1, void* Z, void* Y, void* P, tpmlp::GemmProblem& g1, tpmlp::GemmProblem& g2) {
  // Z_i = X·A_i (+ b1_i) and Y_i = GeLU(Z_i): A = X [n,d] (K-major),
  // B = A_i [d,m_i] (N-major), batched over shards with X shared.
  g1 = tpmlp::GemmProblem{};
  g1.M = static_cast<int>(n);
  g1.N = static_cast<int>(m_i);
  g1.K = static_cast<int>(d);
  g1.batch = t_local;
  g1.A = X;
  g1.B = A;
  g1.C = Z;
  g1.C2 = Y;
  g1.bias = b1;
  g1.sBias = m_i;
  g1.lda = d;
  g1.ldb = m_i;
  g1.ldc = m_i;
  g1.sA = 0;
  g1.sB = d * m_i;
  g1.sC = n * m_i;

  // P_i = Y_i·B_i: A = Y_i [n,m_i] (K-major), B = B_i [m_i,d] (N-major).
  g2 = tpmlp::GemmProblem{};
  g2.M = static_cast<int>(n);
  g2.N = static_cast<int>(d);
  g2.K = static_cast<int>(m_i);
  g2.batch = t_local;
  g2.A = Y;
  g2.B = B;
  g2.C = P;
  g2.lda = m_i;
  g2.ldb = d;
  g2.ldc = d;
  g2.sA = n * m_i;
  g2.sB = m_i * d;
  g2.sC = n * d;
}

size_t fwd_ws_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local, bool bias) {
  if (dt != TPMLP_BF16 || check_mlp_dims(dt, n, d, m_i, t_local) != TPMLP_OK || n == 0) return 0;
  tpmlp::GemmProblem g1, g2;
  fwd_problems(n, d, m_i, t_local, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, g1, g2);
  const tpmlp::GemmKind k1{tpmlp::KMAJ, tpmlp::MNMAJ, bias ? tpmlp::EPI_BIAS_GELU_ZY : tpmlp::EPI_GELU_ZY};
  const tpmlp::GemmKind k2{tpmlp::KMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE};
  const size_t a = tpmlp::gemm_bf16_split_bytes(&g1, 1, k1, nullptr, k1);
  const size_t b = tpmlp::gemm_bf16_split_bytes(&g2, 1, k2, nullptr, k2);
  return a > b ? a : b;
}

// The shard forward with an optional column bias b1 [t_local, m_i] (NULL: none).
int fwd_impl(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local, const void* X,
             const void* A, const void* B, const void* b1, void* Z, void* Y, void* P, void* ws, size_t ws_bytes) {
  int st = check_mlp_dims(dt, n, d, m_i, t_local);
  if (st) return st;
  if (n == 0) return TPMLP_OK;
  st = check_ptrs(dt, {X, A, B, Z, Y, P});
  if (st) return st;
  const size_t need = fwd_ws_bytes(dt, n, d, m_i, t_local, b1 != nullptr);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return TPMLP_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return TPMLP_ERR_ALIGN;
  tpmlp::GemmProblem g1, g2;
  fwd_problems(n, d, m_i, t_local, X, A, B, b1, Z, Y, P, g1, g2);
  const int epi1 = b1 != nullptr ? tpmlp::EPI_BIAS_GELU_ZY : tpmlp::EPI_GELU_ZY;
  if (dt == TPMLP_BF16) {
    st = hip_status(tpmlp::launch_gemm_bf16_ws(g1, tpmlp::KMAJ, tpmlp::MNMAJ, epi1, ws, ws_bytes, stream));
    if (st) return st;
    return hip_status(
        tpmlp::launch_gemm_bf16_ws(g2, tpmlp::KMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE, ws, ws_bytes, stream));
  }
  st = hip_status(gemm(dt, g1, tpmlp::KMAJ, tpmlp::MNMAJ, epi1, stream));
  if (st) return st;
  return hip_status(gemm(dt, g2, tpmlp::KMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE, stream));
}

int reduce_impl(hipStream_t stream, int in_dt, int out_dt, int32_t t, int64_t rows, int64_t cols,
                const void* partials, const void* bias, void* out) {
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return TPMLP_ERR_DTYPE;
  if (t < 1 || rows < 0 || cols < 1) return TPMLP_ERR_SHAPE;
  if (rows > 0 && cols > (int64_t{1} << 62) / rows) return TPMLP_ERR_SHAPE;
  const int64_t count = rows * cols;
  if (count > (int64_t{1} << 62) / t) return TPMLP_ERR_SHAPE;
  if (count == 0) return TPMLP_OK;
  if (partials == nullptr || out == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(partials, elem_size(in_dt)) || !aligned(out, elem_size(out_dt))) return TPMLP_ERR_ALIGN;
  if (bias != nullptr && !aligned(bias, elem_size(out_dt))) return TPMLP_ERR_ALIGN;
  return hip_status(tpmlp::launch_reduce_partials(in_dt, out_dt, t, count, partials, out, bias, cols, stream));
}

}  // namespace

extern "C" {

int tpmlp_abi_version(void) { return TPMLP_ABI_VERSION; }

static_assert(TPMLP_GEMM_TILE_AUTO == tpmlp::TILE_AUTO && TPMLP_GEMM_TILE_256 == tpmlp::TILE_256 &&
                  TPMLP_GEMM_TILE_192 == tpmlp::TILE_192 && TPMLP_GEMM_STREAMK == tpmlp::TILE_STREAMK &&
                  TPMLP_GEMM_TILE_128 == tpmlp::TILE_128,
              "tile policy values");

int tpmlp_set_gemm_tile_policy(int policy) {
  if (policy != TPMLP_GEMM_TILE_AUTO && policy != TPMLP_GEMM_TILE_256 && policy != TPMLP_GEMM_TILE_192 &&
      policy != TPMLP_GEMM_STREAMK && policy != TPMLP_GEMM_TILE_128)
    return TPMLP_ERR_ARG;
  tpmlp::set_gemm_tile_policy(policy);
  return TPMLP_OK;
}

int tpmlp_gemm_tile_policy(void) { return tpmlp::gemm_tile_policy(); }

int tpmlp_last_hip_error(void) { return g_last_hip_error; }

const char* tpmlp_status_string(int status) {
  switch (status) {
    case TPMLP_OK: return "ok";
    case TPMLP_ERR_NULLPTR: return "a required pointer is NULL";
    case TPMLP_ERR_SHAPE: return "invalid shape (non-positive size, uneven shard split, size limit, or t < 2 for sequence parallelism)";
    case TPMLP_ERR_DTYPE: return "unsupported dtype";
    case TPMLP_ERR_ALIGN: return "misaligned pointer or row length (bf16 needs 16-byte bases and rows of a multiple of 8 elements)";
    case TPMLP_ERR_HIP: return "a HIP kernel launch failed";
    case TPMLP_ERR_WORKSPACE: return "workspace missing or too small";
    case TPMLP_ERR_ARG: return "invalid argument";
    case TPMLP_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point's fixed array holds";
    default: return "unknown status";
  }
}

size_t tpmlp_fwd_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  return fwd_ws_bytes(dt, n, d, m_i, t_local, false);
}

size_t tpmlp_fwd_bias_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  return fwd_ws_bytes(dt, n, d, m_i, t_local, true);
}

int tpmlp_fwd(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
              const void* X, const void* A, const void* B, void* Z, void* Y, void* P, void* ws, size_t ws_bytes) {
  return fwd_impl(stream, dt, n, d, m_i, t_local, X, A, B, nullptr, Z, Y, P, ws, ws_bytes);
}

int tpmlp_fwd_bias(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
                   const void* X, const void* A, const void* B, const void* b1, void* Z, void* Y, void* P, void* ws,
                   size_t ws_bytes) {
  int st = check_mlp_dims(dt, n, d, m_i, t_local);
  if (st) return st;
  if (n == 0) return TPMLP_OK;
  st = check_ptrs(dt, {b1});
  if (st) return st;
  return fwd_impl(stream, dt, n, d, m_i, t_local, X, A, B, b1, Z, Y, P, ws, ws_bytes);
}

}  // extern "C"

namespace {

// The backward's four products (pointers may be null for a size query).
void bwd_problems(int64_t n, int64_t d, int64_t m_i, int32_t t_local, const void* X, const void* A,
                  const void* B, const void* Z, const void* Y, const void* G, void* D, float* dA, float* dB,
                  void* dXp, tpmlp::GemmProblem& e, tpmlp::GemmProblem& wb, tpmlp::GemmProblem& wa,
                  tpmlp::GemmProblem& dx) {
  // D_i = (G·B_iᵀ) ⊙ GeLU'(Z_i): A = G [n,d] (K-major), B(k,j) = B_i[j][k]
  // (K-major, ld = d).  Empty (skipped) when n == 0.
  e = tpmlp::GemmProblem{};
  e.M = static_cast<int>(n);
  e.N = static_cast<int>(m_i);
  e.K = static_cast<int>(d);
  e.batch = t_local;
  e.A = G;
  e.B = B;
  e.C = D;
  e.Zin = Z;
  e.lda = d;
  e.ldb = d;
  e.ldc = m_i;
  e.sA = 0;
  e.sB = m_i * d;
  e.sC = n * m_i;

  // dB_i = Y_iᵀ·G: M = m_i, N = d, K = n; A(m,k) = Y_i[k][m] (M-major),
  // B(k,j) = G[k][j] (N-major).  With n == 0 this writes zeros.
  wb = tpmlp::GemmProblem{};
  wb.M = static_cast<int>(m_i);
  wb.N = static_cast<int>(d);
  wb.K = static_cast<int>(n);
  wb.batch = t_local;
  wb.A = Y;
  wb.B = G;
  wb.C = dB;
  wb.lda = m_i;
  wb.ldb = d;
  wb.ldc = d;
  wb.sA = n * m_i;
  wb.sB = 0;
  wb.sC = m_i * d;

  // dA_i = Xᵀ·D_i: M = d, N = m_i, K = n; A(m,k) = X[k][m], B(k,j) = D_i[k][j].
  wa = tpmlp::GemmProblem{};
  wa.M = static_cast<int>(d);
  wa.N = static_cast<int>(m_i);
  wa.K = static_cast<int>(n);
  wa.batch = t_local;
  wa.A = X;
  wa.B = D;
  wa.C = dA;
  wa.lda = d;
  wa.ldb = m_i;
  wa.ldc = m_i;
  wa.sA = 0;
  wa.sB = n * m_i;
  wa.sC = d * m_i;

  // dX_i = D_i·A_iᵀ: M = n, N = d, K = m_i; A = D_i (K-major),
  // B(k,j) = A_i[j][k] (K-major, ld = m_i).  Empty (skipped) when n == 0.
  dx = tpmlp::GemmProblem{};
  dx.M = static_cast<int>(n);
  dx.N = static_cast<int>(d);
  dx.K = static_cast<int>(m_i);
  dx.batch = t_local;
  dx.A = D;
  dx.B = A;
  dx.C = dXp;
  dx.lda = m_i;
  dx.ldb = m_i;
  dx.ldc = d;
  dx.sA = n * m_i;
  dx.sB = d * m_i;
  dx.sC = n * d;
}

const tpmlp::GemmKind kWgrad{tpmlp::MNMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE_F32};
const tpmlp::GemmKind kDgrad1{tpmlp::KMAJ, tpmlp::KMAJ, tpmlp::EPI_GELU_GRAD};
const tpmlp::GemmKind kDgrad2{tpmlp::KMAJ, tpmlp::KMAJ, tpmlp::EPI_STORE};

size_t bwd_ws_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  if (dt != TPMLP_BF16 || check_mlp_dims(dt, n, d, m_i, t_local) != TPMLP_OK) return 0;
  tpmlp::GemmProblem e, wb, wa, dx;
  bwd_problems(n, d, m_i, t_local, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
               nullptr, e, wb, wa, dx);
  const tpmlp::GemmProblem w[2] = {wb, wa};
  const size_t a = tpmlp::gemm_bf16_split_bytes(&e, 1, kDgrad1, nullptr, kDgrad1);
  const size_t b = tpmlp::gemm_bf16_split_bytes(w, 2, kWgrad, &dx, kDgrad2);
  return a > b ? a : b;
}

}  // namespace

extern "C" {

size_t tpmlp_bwd_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  return bwd_ws_bytes(dt, n, d, m_i, t_local);
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the biased backward: the weight-gradient launch's split
// partials (dgrad-1 with the fused column sums is never split), then the
// 128-row chunk column sums of D (db1) and of G (db2).
struct BwdBiasWs {
  size_t split, db1, db2, total;
};

BwdBiasWs bwd_bias_ws(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  BwdBiasWs w{0, 0, 0, 0};
  if (check_mlp_dims(dt, n, d, m_i, t_local) != TPMLP_OK) return w;
  if (dt == TPMLP_BF16) {
    tpmlp::GemmProblem e, wb, wa, dx;
    bwd_problems(n, d, m_i, t_local, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                 nullptr, e, wb, wa, dx);
    const tpmlp::GemmProblem wp[2] = {wb, wa};
    w.split = align256(tpmlp::gemm_bf16_split_bytes(wp, 2, kWgrad, &dx, kDgrad2));
  }
  const int64_t nc = tpmlp::bias_grad_chunks(n);
  w.db1 = align256(static_cast<size_t>(t_local) * static_cast<size_t>(nc) * static_cast<size_t>(m_i) * 4);
  w.db2 = align256(static_cast<size_t>(nc) * static_cast<size_t>(d) * 4);
  w.total = w.split + w.db1 + w.db2;
  return w;
}

// The shard backward; with db1 and db2 (both non-null) also the bias
// gradients db1_i = Σ_rows D_i and db2 = Σ_rows G.
int bwd_impl(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local, const void* X,
             const void* A, const void* B, const void* Z, const void* Y, const void* G, void* D, float* dA, float* dB,
             void* dXp, float* db1, float* db2, void* ws, size_t ws_bytes) {
  int st = check_mlp_dims(dt, n, d, m_i, t_local);
  if (st) return st;
  const bool bias = db1 != nullptr;
  const size_t need = bias ? bwd_bias_ws(dt, n, d, m_i, t_local).total : tpmlp_bwd_workspace_bytes(dt, n, d, m_i, t_local);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return TPMLP_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return TPMLP_ERR_ALIGN;
  if (dA == nullptr || dB == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(dA, wgrad_align(dt)) || !aligned(dB, wgrad_align(dt))) return TPMLP_ERR_ALIGN;
  if (bias && (!aligned(db1, 4) || !aligned(db2, 4))) return TPMLP_ERR_ALIGN;
  if (n > 0) {
    st = check_ptrs(dt, {X, A, B, Z, Y, G, D, dXp});
    if (st) return st;
  }
  tpmlp::GemmProblem e, wb, wa, dx;
  bwd_problems(n, d, m_i, t_local, X, A, B, Z, Y, G, D, dA, dB, dXp, e, wb, wa, dx);
  const tpmlp::GemmKind& wgrad = kWgrad;
  const tpmlp::GemmKind& dgrad1 = kDgrad1;
  const tpmlp::GemmKind& dgrad2 = kDgrad2;
  // the biased backward's workspace regions
  BwdBiasWs bw{0, 0, 0, 0};
  float* ws_db1 = nullptr;
  float* ws_db2 = nullptr;
  void* ws_split = ws;
  size_t split_bytes = ws_bytes;
  if (bias) {
    bw = bwd_bias_ws(dt, n, d, m_i, t_local);
    ws_db1 = reinterpret_cast<float*>(static_cast<char*>(ws) + bw.split);
    ws_db2 = reinterpret_cast<float*>(static_cast<char*>(ws) + bw.split + bw.db1);
    split_bytes = bw.split;
  }
  if (dt == TPMLP_BF16) {
    // Two launches: dgrad-1, then both weight gradients (K = n, the long
    // ones) with dgrad-2 (which also needs D), whose tiles fill the machine
    // around them.  Products that would leave the machine idle run K-split
    // in the workspace.  With the bias gradients, dgrad-1's epilogue also
    // writes the column sums of each 128-row chunk of D ([EFF] §4.2: the
    // bias work fused into the GEMM), summed over the chunks after it.
    if (bias) {
      e.colsum = ws_db1;
      st = hip_status(tpmlp::launch_gemm_bf16_ws(e, tpmlp::KMAJ, tpmlp::KMAJ, tpmlp::EPI_GELU_GRAD_DB, nullptr, 0,
                                                 stream));
      if (st) return st;
      st = hip_status(tpmlp::launch_bias_grad_final(t_local, n, m_i, db1, ws_db1, stream));
    } else {
      st = hip_status(
          tpmlp::launch_gemm_bf16_ws(e, dgrad1.a_order, dgrad1.b_order, dgrad1.epi, ws, ws_bytes, stream));
    }
    if (st) return st;
    const tpmlp::GemmProblem w[2] = {wb, wa};
    st = hip_status(tpmlp::launch_gemm_bf16_group(w, 2, wgrad, &dx, dgrad2, ws_split, split_bytes, stream));
    if (st || !bias) return st;
    return hip_status(tpmlp::launch_bias_grad(dt, 1, n, d, G, db2, ws_db2, stream));
  }
  if (n > 0) {
    st = hip_status(gemm(dt, e, dgrad1.a_order, dgrad1.b_order, dgrad1.epi, stream));
    if (st) return st;
  }
  if (bias) {
    st = hip_status(tpmlp::launch_bias_grad(dt, t_local, n, m_i, D, db1, ws_db1, stream));
    if (st) return st;
    st = hip_status(tpmlp::launch_bias_grad(dt, 1, n, d, G, db2, ws_db2, stream));
    if (st) return st;
  }
  st = hip_status(gemm(dt, wb, wgrad.a_order, wgrad.b_order, wgrad.epi, stream));
  if (st) return st;
  st = hip_status(gemm(dt, wa, wgrad.a_order, wgrad.b_order, wgrad.epi, stream));
  if (st) return st;
  if (n > 0) {
    st = hip_status(gemm(dt, dx, dgrad2.a_order, dgrad2.b_order, dgrad2.epi, stream));
    if (st) return st;
  }
  return TPMLP_OK;
}

}  // namespace

extern "C" {

int tpmlp_bwd(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
              const void* X, const void* A, const void* B, const void* Z, const void* Y,
              const void* G, void* D, float* dA, float* dB, void* dXp, void* ws, size_t ws_bytes) {
  return bwd_impl(stream, dt, n, d, m_i, t_local, X, A, B, Z, Y, G, D, dA, dB, dXp, nullptr, nullptr, ws, ws_bytes);
}

size_t tpmlp_bwd_bias_workspace_bytes(int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local) {
  return bwd_bias_ws(dt, n, d, m_i, t_local).total;
}

int tpmlp_bwd_bias(hipStream_t stream, int dt, int64_t n, int64_t d, int64_t m_i, int32_t t_local,
                   const void* X, const void* A, const void* B, const void* Z, const void* Y, const void* G, void* D,
                   float* dA, float* dB, void* dXp, float* db1, float* db2, void* ws, size_t ws_bytes) {
  if (db1 == nullptr || db2 == nullptr) return TPMLP_ERR_NULLPTR;
  if (t_local > 65535) return TPMLP_ERR_SHAPE;  // the chunk sums' grid
  return bwd_impl(stream, dt, n, d, m_i, t_local, X, A, B, Z, Y, G, D, dA, dB, dXp, db1, db2, ws, ws_bytes);
}

int tpmlp_reduce_partials(hipStream_t stream, int in_dt, int out_dt, int32_t t, int64_t rows,
                          int64_t cols, const void* partials, void* out) {
  return reduce_impl(stream, in_dt, out_dt, t, rows, cols, partials, nullptr, out);
}

int tpmlp_reduce_partials_bias(hipStream_t stream, int in_dt, int out_dt, int32_t t, int64_t rows,
                               int64_t cols, const void* partials, const void* bias, void* out) {
  if (bias == nullptr) return TPMLP_ERR_NULLPTR;
  return reduce_impl(stream, in_dt, out_dt, t, rows, cols, partials, bias, out);
}

size_t tpmlp_bias_grad_workspace_bytes(int32_t t, int64_t rows, int64_t cols) {
  if (t < 1 || rows <= 0 || cols <= 0) return 0;
  return static_cast<size_t>(t) * static_cast<size_t>(tpmlp::bias_grad_chunks(rows)) *
         static_cast<size_t>(cols) * sizeof(float);
}

}  // extern "C"

namespace {

// The checks of tpmlp_bias_grad other than its workspace's.
int bias_grad_check(int dt, int32_t t, int64_t rows, int64_t cols, const void* g, const float* db) {
  if (!valid_dt(dt)) return TPMLP_ERR_DTYPE;
  if (t < 1 || rows < 0 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return TPMLP_ERR_SHAPE;
  if (rows > 0 && cols > (int64_t{1} << 62) / rows) return TPMLP_ERR_SHAPE;
  if (rows * cols > (int64_t{1} << 62) / t) return TPMLP_ERR_SHAPE;
  // launch grid limits: chunk × column-block blocks in x, shards in y
  if (t > 65535 || ((cols + 31) / 32) * tpmlp::bias_grad_chunks(rows) > kMaxDim ||
      (t * cols + 31) / 32 > kMaxDim)
    return TPMLP_ERR_SHAPE;
  if (db == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(db, 4)) return TPMLP_ERR_ALIGN;
  if (rows > 0) {
    if (g == nullptr) return TPMLP_ERR_NULLPTR;
    if (!aligned(g, elem_size(dt))) return TPMLP_ERR_ALIGN;
  }
  return TPMLP_OK;
}

}  // namespace

extern "C" {

int tpmlp_bias_grad(hipStream_t stream, int dt, int32_t t, int64_t rows, int64_t cols, const void* g,
                    float* db, void* ws, size_t ws_bytes) {
  const int st = bias_grad_check(dt, t, rows, cols, g, db);
  if (st) return st;
  if (rows > 0) {
    const size_t need = tpmlp_bias_grad_workspace_bytes(t, rows, cols);
    if (ws == nullptr || ws_bytes < need) return TPMLP_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return TPMLP_ERR_ALIGN;
  }
  return hip_status(tpmlp::launch_bias_grad(dt, t, rows, cols, g, db, static_cast<float*>(ws), stream));
}

}  // extern "C"

// ------------------------------------------------- allocation-free bias gradient
// tpmlp_bias_grad_noalloc keeps the bias gradient's chunk partials in a fixed
// device array of the library instead of a caller's workspace.  Each device
// holds its own copy of the array at its own address: the host-side name
// `scratch` is only a stand-in, so its device address is looked up once per
// device (with that device current) and kept; kernels are only ever given the
// looked-up address.
namespace {

constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[TPMLP_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // the address of `scratch` on each device, or null before the lookup

// The scratch address on the device that runs `stream` (the current device
// for the null stream).  HIP status on failure.
hipError_t scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int tpmlp_bias_grad_noalloc(hipStream_t stream, int dt, int32_t t, int64_t rows, int64_t cols, const void* g,
                            float* db) {
  const int st = bias_grad_check(dt, t, rows, cols, g, db);
  if (st) return st;
  if (tpmlp_bias_grad_workspace_bytes(t, rows, cols) > TPMLP_NOALLOC_SCRATCH_BYTES) return TPMLP_ERR_SCRATCH;
  void* ws = nullptr;
  if (rows > 0) {  // rows == 0 only zeroes db and needs no scratch
    const int hs = hip_status(scratch_for(stream, &ws));
    if (hs) return hs;
  }
  // stage 1 writes every chunk partial that stage 2 reads: nothing needs clearing
  return hip_status(tpmlp::launch_bias_grad(dt, t, rows, cols, g, db, static_cast<float*>(ws), stream));
}

size_t tpmlp_sp_workspace_bytes(int64_t s, int64_t h) {
  if (s <= 0 || h <= 0) return 0;
  return static_cast<size_t>(tpmlp::sp_workspace_floats(s, h)) * sizeof(float);
}

int tpmlp_ln_sp(hipStream_t stream, const tpmlp_sp_args* a) {
  if (a == nullptr) return TPMLP_ERR_NULLPTR;
  if (!valid_dt(a->dt)) return TPMLP_ERR_DTYPE;
  if (a->phase < TPMLP_SP_LN_FWD || a->phase > TPMLP_SP_LN_BWD) return TPMLP_ERR_ARG;
  if (a->t < 2) return TPMLP_ERR_SHAPE;  // sequence parallelism needs TP > 1
  if (a->s < 0 || a->h < 8 || a->row0 < 0) return TPMLP_ERR_SHAPE;
  if (a->s % a->t != 0) return TPMLP_ERR_SHAPE;
  if (a->h % 8 != 0) return TPMLP_ERR_ALIGN;
  if (!(a->p_drop >= 0.0f && a->p_drop < 1.0f)) return TPMLP_ERR_ARG;
  if (!(a->eps > 0.0f)) return TPMLP_ERR_ARG;
  if (a->s == 0) return TPMLP_OK;
  const int es = elem_size(a->dt);
  if (!fits(a->s, a->h, es) || !fits(a->s * a->t, a->h, es)) return TPMLP_ERR_SHAPE;

  tpmlp::SpProblem p{};
  p.phase = a->phase;
  p.dt = a->dt;
  p.t = a->t;
  p.s = a->s;
  p.h = a->h;
  p.row0 = a->row0;
  p.eps = a->eps;
  p.drop_threshold = static_cast<uint32_t>(floor(static_cast<double>(a->p_drop) * 4294967296.0));
  p.keep_scale = static_cast<float>(1.0 / (1.0 - static_cast<double>(a->p_drop)));
  p.seed = a->seed;
  p.x = a->x;
  p.gamma = a->gamma;
  p.beta = a->beta;
  p.ln_out = a->ln_out;
  p.mean = a->mean;
  p.rstd = a->rstd;
  p.partials = a->partials;
  p.out = a->out;
  p.g_out = a->g_out;
  p.dS = a->dS;
  p.dU_partials = a->dU_partials;
  p.dx = a->dx;
  p.dgamma = a->dgamma;
  p.dbeta = a->dbeta;
  p.ws = static_cast<float*>(a->ws);
  p.bias = a->phase == TPMLP_SP_DROPRES_FWD ? a->bias : nullptr;

  const uintptr_t al = 16;
  auto ok = [&](std::initializer_list<const void*> ps) {
    for (const void* q : ps)
      if (q == nullptr) return TPMLP_ERR_NULLPTR;
    for (const void* q : ps)
      if (!aligned(q, al)) return TPMLP_ERR_ALIGN;
    return TPMLP_OK;
  };
  int st = TPMLP_OK;
  switch (a->phase) {
    case TPMLP_SP_LN_FWD:
      st = ok({a->x, a->gamma, a->beta, a->ln_out});
      if (!st && (a->mean == nullptr || a->rstd == nullptr)) st = TPMLP_ERR_NULLPTR;
      if (!st && (!aligned(a->mean, 4) || !aligned(a->rstd, 4))) st = TPMLP_ERR_ALIGN;
      break;
    case TPMLP_SP_DROPRES_FWD:
      st = ok({a->partials, a->x, a->out});
      if (!st && a->bias != nullptr && !aligned(a->bias, al)) st = TPMLP_ERR_ALIGN;
      break;
    case TPMLP_SP_DROPRES_BWD:
      st = ok({a->g_out, a->dS});
      break;
    default:
      st = ok({a->dU_partials, a->g_out, a->x, a->gamma, a->dx});
      if (!st && (a->mean == nullptr || a->rstd == nullptr || a->dgamma == nullptr ||
                  a->dbeta == nullptr))
        st = TPMLP_ERR_NULLPTR;
      if (!st && (!aligned(a->mean, 4) || !aligned(a->rstd, 4) || !aligned(a->dgamma, 4) ||
                  !aligned(a->dbeta, 4)))
        st = TPMLP_ERR_ALIGN;
      if (!st && (a->ws == nullptr || a->ws_bytes < tpmlp_sp_workspace_bytes(a->s, a->h)))
        st = TPMLP_ERR_WORKSPACE;
      if (!st && !aligned(a->ws, 4)) st = TPMLP_ERR_ALIGN;
      break;
  }
  if (st) return st;
  return hip_status(tpmlp::launch_sp(p, stream));
}

}  // extern "C"

// ------------------------------------------------------------------ attention
namespace {

// Shared checks of the attention entry points; fills the core problem.
int attn_core_problem(int dt, int32_t t_local, int64_t s, int64_t b, int32_t nh, int32_t dh, int causal,
                      const uint32_t* mask, tpmlp::AttnProblem& p) {
  if (!valid_dt(dt)) return TPMLP_ERR_DTYPE;
  if (t_local < 1 || s < 0 || b < 1 || nh < 1) return TPMLP_ERR_SHAPE;
  if (dh != 64 && dh != 128) return TPMLP_ERR_SHAPE;
  if (causal != 0 && causal != 1) return TPMLP_ERR_ARG;
  if (s > kMaxDim || b > kMaxDim) return TPMLP_ERR_SHAPE;
  const int64_t n = s * b;
  if (n > kMaxDim) return TPMLP_ERR_SHAPE;
  const int es = elem_size(dt);
  if (!fits(n, static_cast<int64_t>(nh) * 3 * dh, es)) return TPMLP_ERR_SHAPE;  // one shard's qkv
  const int64_t wgs = static_cast<int64_t>(t_local) * b * nh * ((s + 127) / 128);
  const int64_t rows = static_cast<int64_t>(t_local) * b * nh * s;
  if (wgs > kMaxDim || rows > kMaxDim) return TPMLP_ERR_SHAPE;
  if (mask != nullptr) {  // one batch entry's part of the packed mask: s·⌈s/32⌉ words
    if (s * ((s + 31) / 32) * 4 > kMaxDim) return TPMLP_ERR_SHAPE;
    if (!aligned(mask, 4)) return TPMLP_ERR_ALIGN;
  }
  p = tpmlp::AttnProblem{};
  p.dt = dt;
  p.T = t_local;
  p.s = static_cast<int>(s);
  p.b = static_cast<int>(b);
  p.nh = nh;
  p.dh = dh;
  p.causal = causal != 0;
  p.mask = mask;
  return TPMLP_OK;
}

}  // namespace

extern "C" {

int tpmlp_attn_core_fwd(hipStream_t stream, int dt, int32_t t_local, int64_t s, int64_t b, int32_t heads_local,
                        int32_t head_dim, int causal, const uint32_t* mask, const void* qkv, void* o, float* lse) {
  tpmlp::AttnProblem p;
  int st = attn_core_problem(dt, t_local, s, b, heads_local, head_dim, causal, mask, p);
  if (st) return st;
  if (s == 0) return TPMLP_OK;
  st = check_ptrs(dt, {qkv, o});
  if (st) return st;
  if (lse == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(lse, 4)) return TPMLP_ERR_ALIGN;
  p.qkv = qkv;
  p.o = o;
  p.lse = lse;
  return hip_status(tpmlp::launch_attn_fwd(p, stream));
}

size_t tpmlp_attn_mask_words(int64_t b, int64_t s) {
  if (b < 1 || s < 1 || s > kMaxDim || b > kMaxDim) return 0;
  return 2 * static_cast<size_t>(b) * static_cast<size_t>(s) * static_cast<size_t>((s + 31) / 32);
}

int tpmlp_attn_pack_mask(hipStream_t stream, int64_t b, int64_t s, const uint8_t* mask, uint32_t* packed) {
  if (b < 1 || s < 0) return TPMLP_ERR_SHAPE;
  if (s == 0) return TPMLP_OK;
  if (s * ((s + 31) / 32) * 4 > kMaxDim || b * s > kMaxDim) return TPMLP_ERR_SHAPE;
  if (mask == nullptr || packed == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(packed, 4)) return TPMLP_ERR_ALIGN;
  return hip_status(tpmlp::launch_attn_pack_mask(static_cast<int>(b), static_cast<int>(s), mask, packed, stream));
}

size_t tpmlp_attn_bwd_workspace_bytes(int32_t t_local, int64_t s, int64_t b, int32_t heads_local) {
  if (t_local < 1 || s <= 0 || b < 1 || heads_local < 1) return 0;
  return static_cast<size_t>(t_local) * static_cast<size_t>(b) * static_cast<size_t>(heads_local) *
         static_cast<size_t>(s) * sizeof(float);
}

int tpmlp_attn_core_bwd(hipStream_t stream, int dt, int32_t t_local, int64_t s, int64_t b, int32_t heads_local,
                        int32_t head_dim, int causal, const uint32_t* mask, const void* qkv, const void* o,
                        const float* lse, const void* d_o, void* dqkv, void* ws, size_t ws_bytes) {
  tpmlp::AttnProblem p;
  int st = attn_core_problem(dt, t_local, s, b, heads_local, head_dim, causal, mask, p);
  if (st) return st;
  if (s == 0) return TPMLP_OK;
  st = check_ptrs(dt, {qkv, o, d_o, dqkv});
  if (st) return st;
  if (lse == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(lse, 4)) return TPMLP_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < tpmlp_attn_bwd_workspace_bytes(t_local, s, b, heads_local))
    return TPMLP_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return TPMLP_ERR_ALIGN;
  p.qkv = qkv;
  p.o = const_cast<void*>(o);
  p.lse = const_cast<float*>(lse);
  p.dout = d_o;
  p.dqkv = dqkv;
  p.delta = static_cast<float*>(ws);
  return hip_status(tpmlp::launch_attn_bwd(p, stream));
}

}  // extern "C"

namespace {

// The shard forward with an optional QKV column bias bqkv [t_local, 3w] (NULL: none).
int attn_fwd_impl(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                  int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                  const void* Wqkv, const void* Wproj, const void* bqkv, void* QKV, void* O, float* lse, void* P) {
  tpmlp::AttnProblem ap;
  int st = attn_core_problem(dt, t_local, s, b, heads_local, head_dim, causal, mask, ap);
  if (st) return st;
  const int64_t n = s * b, w = static_cast<int64_t>(heads_local) * head_dim;
  st = check_mlp_dims(dt, n, d, 3 * w, t_local);  // X·W_qkv and O·W_proj sizes
  if (st) return st;
  if (s == 0) return TPMLP_OK;
  st = check_ptrs(dt, {X, Wqkv, Wproj, QKV, O, P});
  if (st) return st;
  if (lse == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(lse, 4)) return TPMLP_ERR_ALIGN;
  // QKV_i = X·W_qkv,i: A = X [n,d] (K-major), B = W_qkv,i [d,3w] (N-major)
  tpmlp::GemmProblem g1{};
  g1.M = static_cast<int>(n);
  g1.N = static_cast<int>(3 * w);
  g1.K = static_cast<int>(d);
  g1.batch = t_local;
  g1.A = X;
  g1.B = Wqkv;
  g1.C = QKV;
  g1.lda = d;
  g1.ldb = 3 * w;
  g1.ldc = 3 * w;
  g1.sA = 0;
  g1.sB = d * 3 * w;
  g1.sC = n * 3 * w;
  g1.bias = bqkv;
  g1.sBias = 3 * w;
  st = hip_status(gemm(dt, g1, tpmlp::KMAJ, tpmlp::MNMAJ, bqkv != nullptr ? tpmlp::EPI_BIAS_STORE : tpmlp::EPI_STORE,
                       stream));
  if (st) return st;
  ap.qkv = QKV;
  ap.o = O;
  ap.lse = lse;
  st = hip_status(tpmlp::launch_attn_fwd(ap, stream));
  if (st) return st;
  // P_i = O_i·W_proj,i: A = O_i [n,w] (K-major), B = W_proj,i [w,d] (N-major)
  tpmlp::GemmProblem g2{};
  g2.M = static_cast<int>(n);
  g2.N = static_cast<int>(d);
  g2.K = static_cast<int>(w);
  g2.batch = t_local;
  g2.A = O;
  g2.B = Wproj;
  g2.C = P;
  g2.lda = w;
  g2.ldb = d;
  g2.ldc = d;
  g2.sA = n * w;
  g2.sB = w * d;
  g2.sC = n * d;
  return hip_status(gemm(dt, g2, tpmlp::KMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE, stream));
}

}  // namespace

extern "C" {

int tpmlp_attn_fwd(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                   int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                   const void* Wqkv, const void* Wproj, void* QKV, void* O, float* lse, void* P) {
  return attn_fwd_impl(stream, dt, s, b, d, heads_local, head_dim, t_local, causal, mask, X, Wqkv, Wproj, nullptr,
                       QKV, O, lse, P);
}

int tpmlp_attn_fwd_bias(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                        int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                        const void* Wqkv, const void* Wproj, const void* bqkv, void* QKV, void* O, float* lse,
                        void* P) {
  if (bqkv == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(bqkv, dt == TPMLP_BF16 ? 16 : 4)) return TPMLP_ERR_ALIGN;
  return attn_fwd_impl(stream, dt, s, b, d, heads_local, head_dim, t_local, causal, mask, X, Wqkv, Wproj, bqkv,
                       QKV, O, lse, P);
}

int tpmlp_attn_bwd(hipStream_t stream, int dt, int64_t s, int64_t b, int64_t d, int32_t heads_local,
                   int32_t head_dim, int32_t t_local, int causal, const uint32_t* mask, const void* X,
                   const void* Wqkv, const void* Wproj, const void* QKV, const void* O, const float* lse,
                   const void* G, void* dO, void* dQKV, float* dWqkv, float* dWproj, void* dXp, void* ws,
                   size_t ws_bytes) {
  tpmlp::AttnProblem ap;
  int st = attn_core_problem(dt, t_local, s, b, heads_local, head_dim, causal, mask, ap);
  if (st) return st;
  const int64_t n = s * b, w = static_cast<int64_t>(heads_local) * head_dim;
  st = check_mlp_dims(dt, n, d, 3 * w, t_local);
  if (st) return st;
  if (dWqkv == nullptr || dWproj == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(dWqkv, wgrad_align(dt)) || !aligned(dWproj, wgrad_align(dt))) return TPMLP_ERR_ALIGN;
  if (s > 0) {
    st = check_ptrs(dt, {X, Wqkv, Wproj, QKV, O, G, dO, dQKV, dXp});
    if (st) return st;
    if (lse == nullptr) return TPMLP_ERR_NULLPTR;
    if (!aligned(lse, 4)) return TPMLP_ERR_ALIGN;
    if (ws == nullptr || ws_bytes < tpmlp_attn_bwd_workspace_bytes(t_local, s, b, heads_local))
      return TPMLP_ERR_WORKSPACE;
    if (!aligned(ws, 4)) return TPMLP_ERR_ALIGN;
  }
  // dO_i = G·W_proj,iᵀ: M = n, N = w, K = d; B(k,j) = W_proj,i[j][k] (K-major)
  tpmlp::GemmProblem go{};
  go.M = static_cast<int>(n);
  go.N = static_cast<int>(w);
  go.K = static_cast<int>(d);
  go.batch = t_local;
  go.A = G;
  go.B = Wproj;
  go.C = dO;
  go.lda = d;
  go.ldb = d;
  go.ldc = w;
  go.sA = 0;
  go.sB = w * d;
  go.sC = n * w;
  // dW_proj,i = O_iᵀ·G: M = w, N = d, K = n (zeros when n == 0)
  tpmlp::GemmProblem wp{};
  wp.M = static_cast<int>(w);
  wp.N = static_cast<int>(d);
  wp.K = static_cast<int>(n);
  wp.batch = t_local;
  wp.A = O;
  wp.B = G;
  wp.C = dWproj;
  wp.lda = w;
  wp.ldb = d;
  wp.ldc = d;
  wp.sA = n * w;
  wp.sB = 0;
  wp.sC = w * d;
  // dW_qkv,i = Xᵀ·dQKV_i: M = d, N = 3w, K = n
  tpmlp::GemmProblem wq{};
  wq.M = static_cast<int>(d);
  wq.N = static_cast<int>(3 * w);
  wq.K = static_cast<int>(n);
  wq.batch = t_local;
  wq.A = X;
  wq.B = dQKV;
  wq.C = dWqkv;
  wq.lda = d;
  wq.ldb = 3 * w;
  wq.ldc = 3 * w;
  wq.sA = 0;
  wq.sB = n * 3 * w;
  wq.sC = d * 3 * w;
  // dX_i = dQKV_i·W_qkv,iᵀ: M = n, N = d, K = 3w; B(k,j) = W_qkv,i[j][k] (K-major)
  tpmlp::GemmProblem dx{};
  dx.M = static_cast<int>(n);
  dx.N = static_cast<int>(d);
  dx.K = static_cast<int>(3 * w);
  dx.batch = t_local;
  dx.A = dQKV;
  dx.B = Wqkv;
  dx.C = dXp;
  dx.lda = 3 * w;
  dx.ldb = 3 * w;
  dx.ldc = d;
  dx.sA = n * 3 * w;
  dx.sB = d * 3 * w;
  dx.sC = n * d;

  const tpmlp::GemmKind wgrad{tpmlp::MNMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE_F32};
  const tpmlp::GemmKind dgrad{tpmlp::KMAJ, tpmlp::KMAJ, tpmlp::EPI_STORE};
  ap.qkv = QKV;
  ap.o = const_cast<void*>(O);
  ap.lse = const_cast<float*>(lse);
  ap.dout = dO;
  ap.dqkv = dQKV;
  ap.delta = static_cast<float*>(ws);
  if (dt == TPMLP_BF16) {
    // dW_proj (long) with dO (short), the core, then dW_qkv (long) with dX
    st = hip_status(tpmlp::launch_gemm_bf16_group(&wp, 1, wgrad, &go, dgrad, nullptr, 0, stream));
    if (st) return st;
    if (s > 0) {
      st = hip_status(tpmlp::launch_attn_bwd(ap, stream));
      if (st) return st;
    }
    return hip_status(tpmlp::launch_gemm_bf16_group(&wq, 1, wgrad, &dx, dgrad, nullptr, 0, stream));
  }
  st = hip_status(gemm(dt, wp, wgrad.a_order, wgrad.b_order, wgrad.epi, stream));
  if (st) return st;
  if (s > 0) {
    st = hip_status(gemm(dt, go, dgrad.a_order, dgrad.b_order, dgrad.epi, stream));
    if (st) return st;
    st = hip_status(tpmlp::launch_attn_bwd(ap, stream));
    if (st) return st;
  }
  st = hip_status(gemm(dt, wq, wgrad.a_order, wgrad.b_order, wgrad.epi, stream));
  if (st) return st;
  if (s > 0) st = hip_status(gemm(dt, dx, dgrad.a_order, dgrad.b_order, dgrad.epi, stream));
  return st;
}

size_t tpmlp_vocab_ce_workspace_bytes(int32_t t_local, int64_t n, int64_t v_i) {
  if (t_local < 1 || n <= 0 || v_i <= 0) return 0;
  // a (max, sum) pair of floats per shard, token and 64-column group
  return 2 * static_cast<size_t>(t_local) * static_cast<size_t>(n) * static_cast<size_t>((v_i + 63) / 64) *
         sizeof(float);
}

int tpmlp_vocab_ce_fwd(hipStream_t stream, int dt, int64_t n, int64_t h, int64_t v_i, int32_t t_local,
                       int64_t vocab_start, const void* X, const void* W, const int32_t* targets, void* logits,
                       float* loss, float* row_max, float* row_sum, void* ws, size_t ws_bytes) {
  int st = check_mlp_dims(dt, n, h, v_i, t_local);  // X·W_iᵀ has the first GEMM's sizes
  if (st) return st;
  if (vocab_start < 0) return TPMLP_ERR_ARG;
  if (n == 0) return TPMLP_OK;
  st = check_ptrs(dt, {X, W, logits});
  if (st) return st;
  if (targets == nullptr || loss == nullptr || row_max == nullptr || row_sum == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(targets, 4) || !aligned(loss, 4) || !aligned(row_max, 4) || !aligned(row_sum, 4))
    return TPMLP_ERR_ALIGN;
  if (ws == nullptr || ws_bytes < tpmlp_vocab_ce_workspace_bytes(t_local, n, v_i)) return TPMLP_ERR_WORKSPACE;
  if (!aligned(ws, 8)) return TPMLP_ERR_ALIGN;
  // logits_i = X·W_iᵀ: A = X [n,h] (K-major), B(k,j) = W_i[j][k] (K-major);
  // on the bf16 path its epilogue also takes the row statistics per 64-column group
  tpmlp::GemmProblem g{};
  g.M = static_cast<int>(n);
  g.N = static_cast<int>(v_i);
  g.K = static_cast<int>(h);
  g.batch = t_local;
  g.A = X;
  g.B = W;
  g.C = logits;
  g.lda = h;
  g.ldb = h;
  g.ldc = v_i;
  g.sA = 0;
  g.sB = v_i * h;
  g.sC = n * v_i;
  const bool fused = dt == TPMLP_BF16;
  g.rstats = static_cast<float*>(ws);
  st = hip_status(gemm(dt, g, tpmlp::KMAJ, tpmlp::KMAJ, fused ? tpmlp::EPI_STORE_ROWSTATS : tpmlp::EPI_STORE, stream));
  if (st) return st;
  tpmlp::VocabProblem p{};
  p.stats_done = fused;
  p.dt = dt;
  p.T = t_local;
  p.n = n;
  p.vi = v_i;
  p.start0 = vocab_start;
  p.logits = logits;
  p.target = targets;
  p.stats = static_cast<float*>(ws);
  p.loss = loss;
  p.rmax = row_max;
  p.rsum = row_sum;
  return hip_status(tpmlp::launch_vocab_ce_fwd(p, stream));
}

int tpmlp_vocab_ce_bwd(hipStream_t stream, int dt, int64_t n, int64_t h, int64_t v_i, int32_t t_local,
                       int64_t vocab_start, const void* X, const void* W, const int32_t* targets,
                       const void* logits, const float* row_max, const float* row_sum, const float* g,
                       void* dlogits, float* dW, void* dXp) {
  int st = check_mlp_dims(dt, n, h, v_i, t_local);
  if (st) return st;
  if (vocab_start < 0) return TPMLP_ERR_ARG;
  if (dW == nullptr) return TPMLP_ERR_NULLPTR;
  if (!aligned(dW, wgrad_align(dt))) return TPMLP_ERR_ALIGN;
  if (n > 0) {
    st = check_ptrs(dt, {X, W, logits, dlogits, dXp});
    if (st) return st;
    if (targets == nullptr || row_max == nullptr || row_sum == nullptr || g == nullptr) return TPMLP_ERR_NULLPTR;
    if (!aligned(targets, 4) || !aligned(row_max, 4) || !aligned(row_sum, 4) || !aligned(g, 4))
      return TPMLP_ERR_ALIGN;
    tpmlp::VocabProblem p{};
    p.dt = dt;
    p.T = t_local;
    p.n = n;
    p.vi = v_i;
    p.start0 = vocab_start;
    p.logits = logits;
    p.target = targets;
    p.rmax = const_cast<float*>(row_max);
    p.rsum = const_cast<float*>(row_sum);
    p.g = g;
    p.dlogits = dlogits;
    st = hip_status(tpmlp::launch_vocab_ce_bwd(p, stream));
    if (st) return st;
  }
  // dW_i = dlogits_iᵀ·X: M = v_i, N = h, K = n (zeros when n == 0)
  tpmlp::GemmProblem gw{};
  gw.M = static_cast<int>(v_i);
  gw.N = static_cast<int>(h);
  gw.K = static_cast<int>(n);
  gw.batch = t_local;
  gw.A = dlogits;
  gw.B = X;
  gw.C = dW;
  gw.lda = v_i;
  gw.ldb = h;
  gw.ldc = h;
  gw.sA = n * v_i;
  gw.sB = 0;
  gw.sC = v_i * h;
  st = hip_status(gemm(dt, gw, tpmlp::MNMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE_F32, stream));
  if (st || n == 0) return st;
  // dX_i = dlogits_i·W_i: M = n, N = h, K = v_i; B(k,j) = W_i[k][j] (N-major)
  tpmlp::GemmProblem gx{};
  gx.M = static_cast<int>(n);
  gx.N = static_cast<int>(h);
  gx.K = static_cast<int>(v_i);
  gx.batch = t_local;
  gx.A = dlogits;
  gx.B = W;
  gx.C = dXp;
  gx.lda = v_i;
  gx.ldb = h;
  gx.ldc = h;
  gx.sA = n * v_i;
  gx.sB = v_i * h;
  gx.sC = n * h;
  return hip_status(gemm(dt, gx, tpmlp::KMAJ, tpmlp::MNMAJ, tpmlp::EPI_STORE, stream));
}

}  // extern "C"
