// Sequence-parallel region around the MLP block ([SP] placement diagram and
// f/g operator table; [EFF] §3.5.1 backward chain; [TRAIN] LayerNorm and
// Dropout sections):
//   forward   U = LN(x) (row blocks of all t sequence shards = the AllGather),
//             out = x + dropout_p(Σ_i P_i)   (sum, then the row blocks are the
//                                             ReduceScatter's shards)
//   backward  dS = g_out ⊙ mask / (1-p)      (the MLP's upstream gradient)
//             dx = g_out + LN'(Σ_i dU_i);  dγ = Σ_rows dU⊙x̂;  dβ = Σ_rows dU
//
// All kernels are HBM-bound and work on 8-element (16-B bf16) chunks.  The row
// kernels give one wavefront per row (h ≤ 4096: a lane owns h/512 chunks held
// in registers) and reduce with cross-lane shuffles; the dγ/dβ column sums are
// deterministic: per-block partials in a fixed row order, then a fixed-order
// sum over blocks.
//
// Dropout mask: Philox-4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11), written
// here from the paper's round function: counter (c0..c3) and key (k0,k1) go to
// (hi(M1·c2)^c1^k0, lo(M1·c2), hi(M0·c0)^c3^k1, lo(M0·c0)), the key bumped by
// the Weyl constants between the ten rounds.  Element e = (row0+r)·h + c uses
// word e%4 of the block with counter (e/4 as two 32-bit words, 0, 0) and key =
// seed; it is dropped iff that word < floor(p·2^32).
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int WAVE = 64;
constexpr int SP_THREADS = 256;   // 4 waves
constexpr int LNB_ROWS = 32;      // rows per block in the LN backward

// ------------------------------------------------------------------ Philox
__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  u32x4 o;
  o[0] = c0;
  o[1] = c1;
  o[2] = c2;
  o[3] = c3;
  return o;
}

// Keep bits for the 8 elements e0..e0+7 (e0 % 4 == 0): bit j set = kept.
__device__ __forceinline__ uint32_t keep8(uint64_t e0, uint64_t seed, uint32_t thr) {
  const uint64_t q = e0 >> 2;
  const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
  const u32x4 a = philox10(static_cast<uint32_t>(q), static_cast<uint32_t>(q >> 32), 0u, 0u, k0, k1);
  const u32x4 b = philox10(static_cast<uint32_t>(q + 1), static_cast<uint32_t>((q + 1) >> 32), 0u, 0u, k0, k1);
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bits |= (a[j] >= thr ? 1u : 0u) << j;
    bits |= (b[j] >= thr ? 1u : 0u) << (4 + j);
  }
  return bits;
}

// ------------------------------------------------------------------ 8-element I/O
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(u[q] << 16);
      v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
    }
  } else {
    const f32x4 lo = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 hi = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = lo[q];
      v[4 + q] = hi[q];
    }
  }
}

template <typename T>
__device__ __forceinline__ void add8(const T* p, float (&v)[8]) {
  float w[8];
  load8(p, w);
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] += w[q];
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = f2bf(v[q]);
    *reinterpret_cast<bf16x8*>(p) = o;
  } else {
    f32x4 lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[q] = v[q];
      hi[q] = v[4 + q];
    }
    reinterpret_cast<f32x4*>(p)[0] = lo;
    reinterpret_cast<f32x4*>(p)[1] = hi;
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}

// ------------------------------------------------------------------ LN forward
// One wave per row; lane owns chunks q·64 + lane (q < NQ) of the row.
template <typename T, int NQ>
__global__ __launch_bounds__(SP_THREADS) void ln_fwd_kernel(SpProblem p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (SP_THREADS / WAVE) + (threadIdx.x >> 6);
  if (row >= p.s) return;
  const int nchunk = static_cast<int>(p.h / 8);
  const T* x = static_cast<const T*>(p.x) + row * p.h;
  float v[NQ][8];
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = q * WAVE + lane;
    if (c < nchunk) {
      load8(x + c * 8, v[q]);
#pragma unroll
      for (int k = 0; k < 8; ++k) sum += v[q][k];
    }
  }
  const float inv_h = 1.0f / static_cast<float>(p.h);
  const float mean = wave_sum(sum) * inv_h;
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = q * WAVE + lane;
    if (c < nchunk) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float d = v[q][k] - mean;
        ss += d * d;
      }
    }
  }
  const float var = wave_sum(ss) * inv_h;  // biased variance
  const float rstd = 1.0f / sqrtf(var + p.eps);
  const T* gam = static_cast<const T*>(p.gamma);
  const T* bet = static_cast<const T*>(p.beta);
  T* y = static_cast<T*>(p.ln_out) + row * p.h;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = q * WAVE + lane;
    if (c < nchunk) {
      float g[8], b[8], o[8];
      load8(gam + c * 8, g);
      load8(bet + c * 8, b);
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = fmaf((v[q][k] - mean) * rstd, g[k], b[k]);
      store8(y + c * 8, o);
    }
  }
  if (lane == 0) {
    p.mean[row] = mean;
    p.rstd[row] = rstd;
  }
}

// ------------------------------------------------------------------ dropout + residual
// phase 1: out = x + keep·scale·Σ_i P_i ;  phase 2: dS = g_out·keep·scale
template <typename T, bool FWD>
__global__ __launch_bounds__(SP_THREADS) void dropres_kernel(SpProblem p) {
  const int64_t nchunk = p.s * p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t step = static_cast<int64_t>(gridDim.x) * SP_THREADS;
  for (int64_t ch = static_cast<int64_t>(blockIdx.x) * SP_THREADS + threadIdx.x; ch < nchunk; ch += step) {
    const int64_t e = ch * 8;  // local element index; rows are contiguous
    const uint32_t keep = keep8(static_cast<uint64_t>(p.row0 * p.h + e), p.seed, p.drop_threshold);
    float v[8];
    if constexpr (FWD) {
      const T* part = static_cast<const T*>(p.partials);
      load8(part + e, v);
      for (int i = 1; i < p.t; ++i) add8(part + static_cast<int64_t>(i) * count + e, v);
      float xr[8];
      load8(static_cast<const T*>(p.x) + e, xr);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = xr[k] + (((keep >> k) & 1u) ? v[k] * p.keep_scale : 0.0f);
      store8(static_cast<T*>(p.out) + e, v);
    } else {
      load8(static_cast<const T*>(p.g_out) + e, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = ((keep >> k) & 1u) ? v[k] * p.keep_scale : 0.0f;
      store8(static_cast<T*>(p.dS) + e, v);
    }
  }
}

// ------------------------------------------------------------------ LN backward
// Block b handles rows [b·LNB_ROWS, ...): wave w takes rows b·LNB_ROWS + w + 4k.
// Per row: dU = Σ_i dU_i, x̂ = (x-μ)·rstd, g̃ = dU⊙γ,
// dx = g_out + rstd·(g̃ - mean(g̃) - x̂·mean(g̃⊙x̂)).  Column partials of dU⊙x̂
// and dU accumulate in registers per lane, then the 4 waves are summed in
// fixed order through LDS into ws[b][0|1][h].
template <typename T, int NQ>
__global__ __launch_bounds__(SP_THREADS) void ln_bwd_kernel(SpProblem p) {
  extern __shared__ float colsum[];  // [2][h]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nchunk = static_cast<int>(p.h / 8);
  const int64_t count = p.s * p.h;
  const float inv_h = 1.0f / static_cast<float>(p.h);
  const T* gam = static_cast<const T*>(p.gamma);

  float gq[NQ][8];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = q * WAVE + lane;
    if (c < nchunk) load8(gam + c * 8, gq[q]);
  }
  float dg[NQ][8], db[NQ][8];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int k = 0; k < 8; ++k) dg[q][k] = db[q][k] = 0.f;

  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * LNB_ROWS;
  for (int rr = wave; rr < LNB_ROWS; rr += SP_THREADS / WAVE) {
    const int64_t row = r_begin + rr;
    if (row >= p.s) break;
    const float mu = p.mean[row], rs = p.rstd[row];
    const T* dUp = static_cast<const T*>(p.dU_partials) + row * p.h;
    const T* xr = static_cast<const T*>(p.x) + row * p.h;
    float du[NQ][8], xh[NQ][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = q * WAVE + lane;
      if (c < nchunk) {
        load8(dUp + c * 8, du[q]);
        for (int i = 1; i < p.t; ++i) add8(dUp + static_cast<int64_t>(i) * count + c * 8, du[q]);
        load8(xr + c * 8, xh[q]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          xh[q][k] = (xh[q][k] - mu) * rs;
          const float gt = du[q][k] * gq[q][k];
          s1 += gt;
          s2 += gt * xh[q][k];
          dg[q][k] += du[q][k] * xh[q][k];
          db[q][k] += du[q][k];
        }
      }
    }
    const float m1 = wave_sum(s1) * inv_h, m2 = wave_sum(s2) * inv_h;
    const T* go = static_cast<const T*>(p.g_out) + row * p.h;
    T* dx = static_cast<T*>(p.dx) + row * p.h;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c = q * WAVE + lane;
      if (c < nchunk) {
        float o[8];
        load8(go + c * 8, o);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float gt = du[q][k] * gq[q][k];
          o[k] += rs * (gt - m1 - xh[q][k] * m2);
        }
        store8(dx + c * 8, o);
      }
    }
  }
  // Column partials of the 4 waves, summed through LDS in the fixed order
  // ((w0 + w1) + w2) + w3, then written to this block's workspace slot.
  const int h = static_cast<int>(p.h);
  for (int w = 0; w < SP_THREADS / WAVE; ++w) {
    if (wave == w) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int c = q * WAVE + lane;
        if (c < nchunk) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            float* g = &colsum[c * 8 + k];
            float* b = &colsum[h + c * 8 + k];
            *g = w ? *g + dg[q][k] : dg[q][k];
            *b = w ? *b + db[q][k] : db[q][k];
          }
        }
      }
    }
    __syncthreads();
  }
  float* ws = p.ws + static_cast<int64_t>(blockIdx.x) * 2 * h;
  for (int j = threadIdx.x; j < 2 * h; j += SP_THREADS) ws[j] = colsum[j];
}

// dγ[j] = Σ_b ws[b][0][j], dβ[j] = Σ_b ws[b][1][j], b in increasing order.
__global__ __launch_bounds__(SP_THREADS) void colsum_kernel(const float* __restrict__ ws, int64_t nblk,
                                                            int64_t h, float* __restrict__ dgamma,
                                                            float* __restrict__ dbeta) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * SP_THREADS + threadIdx.x;
  if (j >= 2 * h) return;
  float s = 0.f;
  for (int64_t b = 0; b < nblk; ++b) s += ws[b * 2 * h + j];
  if (j < h) dgamma[j] = s;
  else dbeta[j - h] = s;
}

template <typename T, int NQ>
hipError_t launch_nq(const SpProblem& p, hipStream_t stream) {
  const int rows_per_block = SP_THREADS / WAVE;
  switch (p.phase) {
    case 0: {
      const int64_t blocks = (p.s + rows_per_block - 1) / rows_per_block;
      hipLaunchKernelGGL((ln_fwd_kernel<T, NQ>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0,
                         stream, p);
      return hipGetLastError();
    }
    case 1:
    case 2: {
      const int64_t nchunk = p.s * p.h / 8;
      int64_t blocks = (nchunk + SP_THREADS - 1) / SP_THREADS;
      if (blocks > 16384) blocks = 16384;
      if (p.phase == 1)
        hipLaunchKernelGGL((dropres_kernel<T, true>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((dropres_kernel<T, false>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS),
                           0, stream, p);
      return hipGetLastError();
    }
    default: {
      const int64_t nblk = sp_ln_bwd_row_blocks(p.s);
      const size_t lds = 2 * static_cast<size_t>(p.h) * sizeof(float);
      hipLaunchKernelGGL((ln_bwd_kernel<T, NQ>), dim3(static_cast<unsigned>(nblk)), dim3(SP_THREADS), lds,
                         stream, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t cb = (2 * p.h + SP_THREADS - 1) / SP_THREADS;
      hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>(cb)), dim3(SP_THREADS), 0, stream, p.ws,
                         nblk, p.h, p.dgamma, p.dbeta);
      return hipGetLastError();
    }
  }
}

template <typename T>
hipError_t launch_dt(const SpProblem& p, hipStream_t stream) {
  const int64_t nq = (p.h / 8 + WAVE - 1) / WAVE;
  if (nq <= 1) return launch_nq<T, 1>(p, stream);
  if (nq <= 2) return launch_nq<T, 2>(p, stream);
  if (nq <= 4) return launch_nq<T, 4>(p, stream);
  return launch_nq<T, 8>(p, stream);
}

}  // namespace

int64_t sp_ln_bwd_row_blocks(int64_t s) { return (s + LNB_ROWS - 1) / LNB_ROWS; }

hipError_t launch_sp(const SpProblem& p, hipStream_t stream) {
  if (p.s <= 0) return hipSuccess;
  if (p.dt == 1) return launch_dt<bf16>(p, stream);
  return launch_dt<float>(p, stream);
}

}  // namespace tpmlp
