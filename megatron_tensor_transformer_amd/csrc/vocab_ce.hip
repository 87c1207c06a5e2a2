// Vocabulary-parallel cross-entropy ([SENSE] §2.2.2, Eq. (3) and (4)): the
// shards' logits x [T][n][V_i] (logit layer, the GEMM core) never leave their
// shard; each shard reduces its columns to three numbers per token, which are
// combined by a max and two sums, the three small all-reduces of the pages:
//   shard i:  m_i = max_k x_k,  s_i = Σ_k exp(x_k − m_i),  τ_i = x_target or 0
//   combine:  m = max_i m_i,  S = Σ_i s_i·exp(m_i − m),  τ = Σ_i τ_i,
//             loss = ln S + m − τ
// Backward: dx_k = g·(exp(x_k − m)/S − [k = target]).
//
// All three kernels are HBM-bound.  Statistics: one wave per (shard, token)
// row, 16-B loads, a per-lane online max/sum (rescaled only when a lane's
// maximum grows), then a fixed-order wave reduction of the (max, sum) pairs.
// Combine: one thread per token, shards in order.  Backward: 8 elements per
// thread, the row's (m, S, g, target) read once per row segment.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int CT = 256;  // 4 waves, one row each

template <typename T>
__device__ __forceinline__ void load8v(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(u[q] << 16);
      v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
    }
  } else {
    const f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = lo[q];
      v[4 + q] = hi[q];
    }
  }
}

template <typename T>
__device__ __forceinline__ float ld1v(const T* p) {
  if constexpr (sizeof(T) == 2) return bf2f(*p);
  else return *p;
}

// (m, s) ⊕ (m', s'): the pair of the union, rescaled to the larger maximum
__device__ __forceinline__ void merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

// Statistics of row (shard i, token r): m_i, s_i, τ_i into stats[3][T][n].
// VEC: the row is 16-B aligned with V_i % 8 == 0 (else element by element).
template <typename T, bool VEC>
__global__ __launch_bounds__(CT) void ce_stats_kernel(const T* __restrict__ x, const int* __restrict__ target,
                                                      float* __restrict__ stats, int Tn, int64_t n, int64_t vi,
                                                      int64_t start0) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (CT / 64) + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(Tn) * n) return;
  const int64_t i = row / n, r = row - i * n;
  const T* xr = x + row * vi;
  float m = -INFINITY, s = 0.f;
  if constexpr (VEC) {
    for (int64_t c = static_cast<int64_t>(lane) * 8; c < vi; c += 64 * 8) {
      float v[8];
      load8v(xr + c, v);
      float cm = v[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) cm = fmaxf(cm, v[k]);
      if (cm > m) {
        s *= __expf(m - cm);
        m = cm;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s += __expf(v[k] - m);
    }
  } else {
    for (int64_t c = lane; c < vi; c += 64) {
      const float v = ld1v(xr + c);
      if (v > m) {
        s *= __expf(m - v);
        m = v;
      }
      s += __expf(v - m);
    }
  }
  // fixed-order butterfly over the wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    merge(m, s, m2, s2);
  }
  if (lane == 0) {
    const int64_t k = static_cast<int64_t>(target[r]) - (start0 + i * vi);
    const float tau = (k >= 0 && k < vi) ? ld1v(xr + k) : 0.f;
    const int64_t tn = static_cast<int64_t>(Tn) * n;
    stats[row] = m;
    stats[tn + row] = s;
    stats[2 * tn + row] = tau;
  }
}

// Combine the shards' statistics of token r in shard order; loss, and the
// row's max and sum for the backward.
__global__ __launch_bounds__(CT) void ce_combine_kernel(const float* __restrict__ stats, float* __restrict__ loss,
                                                        float* __restrict__ rmax, float* __restrict__ rsum, int Tn,
                                                        int64_t n) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * CT + threadIdx.x;
  if (r >= n) return;
  const int64_t tn = static_cast<int64_t>(Tn) * n;
  float m = -INFINITY;
  for (int i = 0; i < Tn; ++i) m = fmaxf(m, stats[i * n + r]);
  float S = 0.f, tau = 0.f;
  for (int i = 0; i < Tn; ++i) {
    S += stats[tn + i * n + r] * __expf(stats[i * n + r] - m);
    tau += stats[2 * tn + i * n + r];
  }
  loss[r] = logf(S) + m - tau;
  rmax[r] = m;
  rsum[r] = S;
}

// dx[i][r][k] = g_r·(exp(x − m_r)/S_r − [k = target_r − start_i]); 8 elements
// per thread (VEC) or one.
template <typename T, bool VEC>
__global__ __launch_bounds__(CT) void ce_bwd_kernel(const T* __restrict__ x, const int* __restrict__ target,
                                                    const float* __restrict__ rmax, const float* __restrict__ rsum,
                                                    const float* __restrict__ g, T* __restrict__ dx, int Tn,
                                                    int64_t n, int64_t vi, int64_t start0) {
  constexpr int W = VEC ? 8 : 1;
  const int64_t per_row = (vi + W - 1) / W;
  const int64_t total = static_cast<int64_t>(Tn) * n * per_row;
  const int64_t step = static_cast<int64_t>(gridDim.x) * CT;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * CT + threadIdx.x; e < total; e += step) {
    const int64_t row = e / per_row, c = (e - row * per_row) * W;
    const int64_t i = row / n, r = row - i * n;
    const float m = rmax[r], inv = 1.0f / rsum[r], gr = g[r];
    const int64_t k = static_cast<int64_t>(target[r]) - (start0 + i * vi);
    const T* xr = x + row * vi + c;
    T* dr = dx + row * vi + c;
    if constexpr (VEC) {
      float v[8];
      load8v(xr, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = gr * (__expf(v[q] - m) * inv - (c + q == k ? 1.f : 0.f));
      if constexpr (sizeof(T) == 2) {
        bf16x8 o;
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = f2bf(v[q]);
        *reinterpret_cast<bf16x8*>(dr) = o;
      } else {
        f32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lo[q] = v[q];
          hi[q] = v[4 + q];
        }
        reinterpret_cast<f32x4*>(dr)[0] = lo;
        reinterpret_cast<f32x4*>(dr)[1] = hi;
      }
    } else {
      const float v = gr * (__expf(ld1v(xr) - m) * inv - (c == k ? 1.f : 0.f));
      if constexpr (sizeof(T) == 2) *dr = f2bf(v);
      else *dr = v;
    }
  }
}

template <typename T>
hipError_t run_fwd(const VocabProblem& p, hipStream_t stream) {
  const T* x = static_cast<const T*>(p.logits);
  const int64_t rows = static_cast<int64_t>(p.T) * p.n;
  const bool vec = p.vi % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0;
  const unsigned blocks = static_cast<unsigned>((rows + CT / 64 - 1) / (CT / 64));
  if (vec)
    hipLaunchKernelGGL((ce_stats_kernel<T, true>), dim3(blocks), dim3(CT), 0, stream, x, p.target, p.stats, p.T, p.n,
                       p.vi, p.start0);
  else
    hipLaunchKernelGGL((ce_stats_kernel<T, false>), dim3(blocks), dim3(CT), 0, stream, x, p.target, p.stats, p.T,
                       p.n, p.vi, p.start0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ce_combine_kernel, dim3(static_cast<unsigned>((p.n + CT - 1) / CT)), dim3(CT), 0, stream,
                     p.stats, p.loss, p.rmax, p.rsum, p.T, p.n);
  return hipGetLastError();
}

template <typename T>
hipError_t run_bwd(const VocabProblem& p, hipStream_t stream) {
  const T* x = static_cast<const T*>(p.logits);
  T* dx = static_cast<T*>(p.dlogits);
  const bool vec = p.vi % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dx) % 16 == 0;
  const int64_t W = vec ? 8 : 1;
  const int64_t total = static_cast<int64_t>(p.T) * p.n * ((p.vi + W - 1) / W);
  int64_t blocks = (total + CT - 1) / CT;
  if (blocks > 16384) blocks = 16384;
  if (vec)
    hipLaunchKernelGGL((ce_bwd_kernel<T, true>), dim3(static_cast<unsigned>(blocks)), dim3(CT), 0, stream, x,
                       p.target, p.rmax, p.rsum, p.g, dx, p.T, p.n, p.vi, p.start0);
  else
    hipLaunchKernelGGL((ce_bwd_kernel<T, false>), dim3(static_cast<unsigned>(blocks)), dim3(CT), 0, stream, x,
                       p.target, p.rmax, p.rsum, p.g, dx, p.T, p.n, p.vi, p.start0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_vocab_ce_fwd(const VocabProblem& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  return p.dt == 1 ? run_fwd<bf16>(p, stream) : run_fwd<float>(p, stream);
}

hipError_t launch_vocab_ce_bwd(const VocabProblem& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  return p.dt == 1 ? run_bwd<bf16>(p, stream) : run_bwd<float>(p, stream);
}

}  // namespace tpmlp
