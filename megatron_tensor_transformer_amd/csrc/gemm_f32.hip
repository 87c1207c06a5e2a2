// fp32 GEMM for the fp32 path of the MLP shard and of the other layer shards
// (the single-card numeric-alignment path): C[M,N] = A[M,K]·B[K,N] with fp32
// inputs, fp32 products and fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x2_f32), with the same operand orders and epilogues as the
// bf16 core.
//
// A 256-thread workgroup computes a 128×128 tile, each of its 4 waves a 64×64
// quarter as 2×2 blocks of 32×32 (64 accumulators per lane).  K advances 16
// at a time.  Operand tiles are staged through LDS in the operand's own
// memory order, so the global→LDS copy is a straight, coalesced copy of
// 4-byte elements with a bounds check per element: any shape and any 4-byte
// alignment is accepted, down to the 3×4 worked example.  The next K step's
// elements are loaded into registers while the current step's products run,
// and written to the other LDS stage after them (one barrier per step).
//
// Within a K step of 16 the matrix core's two k positions are assigned so
// that lane half h (lanes 32h..32h+31) covers k = 8h .. 8h+7: MFMA kk sums
// over k ∈ {kk, 8 + kk}.  A K-major operand's fragment is then 8 contiguous
// values of a row (two 16-B LDS reads); an M- or N-major operand's is 8
// single reads of consecutive addresses across the lanes.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int BM = 128, BN = 128, BK = 16, NT = 256;
constexpr int KP = BK + 4;   // K-major LDS row: 16 values + 4 pad (conflict-free 16-B reads)
constexpr int GM = 8;        // tile rows per group of the tile order (shared B panels in L2)

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

// LDS floats of one operand tile in the given order: [rows][KP] K-major,
// [BK][rows] M/N-major.
template <int O>
constexpr int tile_floats() {
  return O == KMAJ ? BM * KP : BK * BM;
}

// Load this thread's 8 elements of an operand tile (rows r0.., k k0..) into
// registers; out-of-range elements are zero.  K-major: element q is row
// 16q + t/16, k t%16 (16 lanes read a row's 64 contiguous bytes); M/N-major:
// row t%128, k 2q + t/128 (lanes read consecutive rows of one k).
template <int O>
__device__ __forceinline__ void load_stage(const float* __restrict__ P, int64_t ld, int rows, int K, int r0, int k0,
                                           float (&v)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int r, k;
    if constexpr (O == KMAJ) {
      r = 16 * q + (t >> 4);
      k = t & 15;
    } else {
      r = t & 127;
      k = 2 * q + (t >> 7);
    }
    const int gr = r0 + r, gk = k0 + k;
    v[q] = 0.f;
    if (gr < rows && gk < K)
      v[q] = O == KMAJ ? P[static_cast<int64_t>(gr) * ld + gk] : P[static_cast<int64_t>(gk) * ld + gr];
  }
}

template <int O>
__device__ __forceinline__ void store_stage(float* __restrict__ s, const float (&v)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if constexpr (O == KMAJ) s[(16 * q + (t >> 4)) * KP + (t & 15)] = v[q];
    else s[(2 * q + (t >> 7)) * BM + (t & 127)] = v[q];
  }
}

// The 8 fragment values of rows r0 + lane%32 for this lane's half of the K
// step (k = 8h + kk, kk = 0..7).
template <int O>
__device__ __forceinline__ void read_frag(const float* __restrict__ s, int r0, int lane, float (&f)[8]) {
  const int r = r0 + (lane & 31), h = lane >> 5;
  if constexpr (O == KMAJ) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(s + r * KP + 8 * h);
    const f32x4 y = *reinterpret_cast<const f32x4*>(s + r * KP + 8 * h + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = x[e];
      f[4 + e] = y[e];
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) f[kk] = s[(8 * h + kk) * BM + r];
  }
}

template <int AO, int BO, int EPI>
__global__ __launch_bounds__(NT, 2) void gemm_f32_kernel(F32Args a) {
  __shared__ __attribute__((aligned(16))) float As[2][tile_floats<AO>()];
  __shared__ __attribute__((aligned(16))) float Bs[2][tile_floats<BO>()];
  // grouped tile order: GM tile rows share their B panels while resident
  const int tile = blockIdx.x, batch = blockIdx.y;
  const int per_group = GM * a.tiles_n, g = tile / per_group, first = g * GM;
  const int gsize = a.tiles_m - first < GM ? a.tiles_m - first : GM;
  const int in = tile - g * per_group;
  const int tm = first + in % gsize, tn = in / gsize;
  const int m0 = tm * BM, n0 = tn * BN;
  const float* A = a.A + batch * a.sA;
  const float* B = a.B + batch * a.sB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  float va[8], vb[8];
  load_stage<AO>(A, a.lda, a.M, a.K, m0, 0, va);
  load_stage<BO>(B, a.ldb, a.N, a.K, n0, 0, vb);
  store_stage<AO>(As[0], va);
  store_stage<BO>(Bs[0], vb);
  __syncthreads();

  const int steps = (a.K + BK - 1) / BK;
  for (int s = 0; s < steps; ++s) {
    const int st = s & 1;
    const bool more = s + 1 < steps;
    if (more) {
      load_stage<AO>(A, a.lda, a.M, a.K, m0, (s + 1) * BK, va);
      load_stage<BO>(B, a.ldb, a.N, a.K, n0, (s + 1) * BK, vb);
    }
    float fa[2][8], fb[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) read_frag<AO>(As[st], wm + 32 * i, lane, fa[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) read_frag<BO>(Bs[st], wn + 32 * j, lane, fb[j]);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk], fb[j][kk], acc[i][j], 0, 0, 0);
    if (more) {
      // the other stage was last read in step s − 1, before this step's barrier
      store_stage<AO>(As[st ^ 1], va);
      store_stage<BO>(Bs[st ^ 1], vb);
    }
    __syncthreads();
  }

  // lane L of block (i, j): column 32j + L%32, rows 32i + 8(v/4) + 4(L/32) + v%4
  const int64_t cb = static_cast<int64_t>(batch) * a.sC;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn + 32 * j + (lane & 31);
    if (col >= a.N) continue;
    float bv = 0.f;
    if constexpr (EPI == EPI_BIAS_GELU_ZY || EPI == EPI_BIAS_STORE)
      bv = a.bias[static_cast<int64_t>(batch) * a.sBias + col];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= a.M) continue;
        const int64_t off = cb + static_cast<int64_t>(row) * a.ldc + col;
        const float x = acc[i][j][v] + bv;
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
  k.tiles_m = (p.M + BM - 1) / BM;
  k.tiles_n = (p.N + BN - 1) / BN;
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
