// fp32 GEMM for the fp32 path of the MLP shard (parity-grade accuracy, not the
// throughput path): C[M,N] = A[M,K]·B[K,N], fp32 inputs, fp32 FMA accumulation,
// the same operand orders and epilogues as the bf16 core.
//
// 64×64 tile, K step 16, 256 threads each computing a 4×4 block; operands are
// staged through LDS with predicated loads so any shape (down to the 3×4
// worked example) is handled.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int TM = 64, TN = 64, TK = 16, NT = 256;

struct F32Args {
  const float* A;
  const float* B;
  float* C;
  float* C2;
  const float* Zin;
  const float* bias;
  int64_t sBias;
  int M, N, K;
  int tiles_m, tiles_n;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
};

template <int AO, int BO, int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(F32Args a) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  const int tile = blockIdx.x, batch = blockIdx.y;
  const int tm = tile / a.tiles_n, tn = tile % a.tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;
  const float* A = a.A + batch * a.sA;
  const float* B = a.B + batch * a.sB;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += TK) {
    // 64×16 elements per operand, 4 per thread.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = threadIdx.x + q * NT;
      int r, k;
      if (AO == KMAJ) { r = e / TK; k = e % TK; } else { k = e / TM; r = e % TM; }
      const int gr = m0 + r, gk = k0 + k;
      float v = 0.0f;
      if (gr < a.M && gk < a.K)
        v = AO == KMAJ ? A[static_cast<int64_t>(gr) * a.lda + gk] : A[static_cast<int64_t>(gk) * a.lda + gr];
      As[k][r] = v;
      if (BO == KMAJ) { r = e / TK; k = e % TK; } else { k = e / TN; r = e % TN; }
      const int gc = n0 + r, gk2 = k0 + k;
      float w = 0.0f;
      if (gc < a.N && gk2 < a.K)
        w = BO == KMAJ ? B[static_cast<int64_t>(gc) * a.ldb + gk2] : B[static_cast<int64_t>(gk2) * a.ldb + gc];
      Bs[k][r] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

  const int64_t cb = static_cast<int64_t>(batch) * a.sC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= a.N) continue;
      const int64_t off = cb + static_cast<int64_t>(row) * a.ldc + col;
      float x = acc[i][j];
      if constexpr (EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE)
        x += a.bias[static_cast<int64_t>(batch) * a.sBias + col];
      if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_BIAS_STORE) {
        a.C[off] = x;
      } else if constexpr (EPI == EPI_GELU_ZY || EPI == EPI_BIAS_GELU_ZY) {
        a.C[off] = x;
        a.C2[off] = gelu_precise(x);
      } else {
        a.C[off] = x * gelu_grad_precise(a.Zin[off]);
      }
    }
  }
}

template <int AO, int BO, int EPI>
hipError_t launch_t(const F32Args& k, int batch, hipStream_t stream) {
  dim3 grid(k.tiles_m * k.tiles_n, batch);
  hipLaunchKernelGGL((gemm_f32_kernel<AO, BO, EPI>), grid, dim3(NT), 0, stream, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(const GemmProblem& p, int a_order, int b_order, int epi,
                           hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
  F32Args k;
  k.A = static_cast<const float*>(p.A);
  k.B = static_cast<const float*>(p.B);
  k.C = static_cast<float*>(p.C);
  k.C2 = static_cast<float*>(p.C2);
  k.Zin = static_cast<const float*>(p.Zin);
  k.bias = static_cast<const float*>(p.bias);
  k.sBias = p.sBias;
  k.M = p.M;
  k.N = p.N;
  k.K = p.K;
  k.tiles_m = (p.M + TM - 1) / TM;
  k.tiles_n = (p.N + TN - 1) / TN;
  k.lda = p.lda;
  k.ldb = p.ldb;
  k.ldc = p.ldc;
  k.sA = p.sA;
  k.sB = p.sB;
  k.sC = p.sC;
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_GELU_ZY)
    return launch_t<KMAJ, MNMAJ, EPI_GELU_ZY>(k, p.batch, stream);
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_BIAS_GELU_ZY)
    return launch_t<KMAJ, MNMAJ, EPI_BIAS_GELU_ZY>(k, p.batch, stream);
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_STORE)
    return launch_t<KMAJ, MNMAJ, EPI_STORE>(k, p.batch, stream);
  if (a_order == KMAJ && b_order == MNMAJ && epi == EPI_BIAS_STORE)
    return launch_t<KMAJ, MNMAJ, EPI_BIAS_STORE>(k, p.batch, stream);
  if (a_order == KMAJ && b_order == KMAJ && epi == EPI_GELU_GRAD)
    return launch_t<KMAJ, KMAJ, EPI_GELU_GRAD>(k, p.batch, stream);
  if (a_order == KMAJ && b_order == KMAJ && epi == EPI_STORE)
    return launch_t<KMAJ, KMAJ, EPI_STORE>(k, p.batch, stream);
  if (a_order == MNMAJ && b_order == MNMAJ && epi == EPI_STORE_F32)
    return launch_t<MNMAJ, MNMAJ, EPI_STORE_F32>(k, p.batch, stream);
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
