// Vocabulary-parallel cross-entropy ([SENSE] §2.2.2, Eq. (3) and (4)): the
// shards' logits x [T][n][V_i] (logit layer, the GEMM core) never leave their
// shard; each shard reduces its columns to three numbers per token, which are
// combined by a max and two sums, the three small all-reduces of the pages:
//   shard i:  m_i = max_k x_k,  s_i = Σ_k exp(x_k − m_i),  τ_i = x_target or 0
//   combine:  m = max_i m_i,  S = Σ_i s_i·exp(m_i − m),  τ = Σ_i τ_i,
//             loss = ln S + m − τ
// Backward: dx_k = g·(exp(x_k − m)/S − [k = target]).
//
// The statistics are taken per row and 64-column group of a shard's logits:
// on the bf16 path by the logit GEMM's epilogue from its accumulators as they
// are stored (the logits are then never re-read for them), on the fp32 path
// by a separate kernel.  The combine takes all groups of all shards (the
// shards' max and sums are the same max and sums over more terms, [SENSE]
// Eq. (3)/(4)): one wave per token, a per-lane online max/sum over the groups
// in a fixed order, then a fixed-order butterfly; lane 0 adds the target logit
// of the shard that owns it.  Backward: 8 elements per thread, the row's
// (m, S, g, target) read once per row segment.  All are HBM-bound.
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

// Statistics of row (shard i, token r) over column group g (columns 64g ..
// 64g+63 of the shard): (max, Σ exp(x − max)) into stats[i][r][g].  One thread
// per group; the fp32 path's counterpart of the bf16 GEMM epilogue.
template <typename T>
__global__ __launch_bounds__(CT) void ce_group_stats_kernel(const T* __restrict__ x, float* __restrict__ stats,
                                                            int Tn, int64_t n, int64_t vi, int64_t ng) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * CT + threadIdx.x;
  if (idx >= static_cast<int64_t>(Tn) * n * ng) return;
  const int64_t row = idx / ng, g = idx - row * ng;
  const T* xr = x + row * vi;
  const int64_t c0 = 64 * g, c1 = c0 + 64 < vi ? c0 + 64 : vi;
  float m = -INFINITY, s = 0.f;
  for (int64_t c = c0; c < c1; ++c) {
    const float v = ld1v(xr + c);
    if (v > m) {
      s *= __expf(m - v);
      m = v;
    }
    s += __expf(v - m);
  }
  stats[2 * idx] = m;
  stats[2 * idx + 1] = s;
}

// Token r: combine the (max, sum) pairs of every group of every shard, in
// order, add the target logit of the shard that owns the target; loss, and
// the row's max and sum for the backward.  One wave per token.
template <typename T>
__global__ __launch_bounds__(CT) void ce_combine_kernel(const float* __restrict__ stats, const T* __restrict__ x,
                                                        const int* __restrict__ target, float* __restrict__ loss,
                                                        float* __restrict__ rmax, float* __restrict__ rsum, int Tn,
                                                        int64_t n, int64_t vi, int64_t ng, int64_t start0) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (CT / 64) + (threadIdx.x >> 6);
  if (r >= n) return;
  float m = -INFINITY, s = 0.f;
  const int64_t per = Tn * ng;  // pairs of token r: shard i's groups at (i·n + r)·ng
  for (int64_t k = lane; k < per; k += 64) {
    const int64_t i = k / ng, g = k - i * ng;
    const float* p = stats + ((i * n + r) * ng + g) * 2;
    merge(m, s, p[0], p[1]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    merge(m, s, m2, s2);
  }
  if (lane == 0) {
    const int64_t gt = static_cast<int64_t>(target[r]) - start0;  // column in the resident shards' vocabulary
    float tau = 0.f;
    if (gt >= 0 && gt < static_cast<int64_t>(Tn) * vi) {
      const int64_t i = gt / vi, k = gt - i * vi;
      tau = ld1v(x + (i * n + r) * vi + k);
    }
    loss[r] = logf(s) + m - tau;
    rmax[r] = m;
    rsum[r] = s;
  }
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
  const int64_t ng = (p.vi + 63) / 64;
  if (!p.stats_done) {
    const int64_t groups = static_cast<int64_t>(p.T) * p.n * ng;
    hipLaunchKernelGGL((ce_group_stats_kernel<T>), dim3(static_cast<unsigned>((groups + CT - 1) / CT)), dim3(CT), 0,
                       stream, x, p.stats, p.T, p.n, p.vi, ng);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ce_combine_kernel<T>), dim3(static_cast<unsigned>((p.n + CT / 64 - 1) / (CT / 64))), dim3(CT),
                     0, stream, p.stats, x, p.target, p.loss, p.rmax, p.rsum, p.T, p.n, p.vi, ng, p.start0);
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
