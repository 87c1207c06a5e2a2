// out = Σ_{i<t} partials[i]: the one-GPU stand-in for the tensor-parallel
// all-reduce after the row-parallel GEMM (forward) and of the column-parallel
// input gradient (backward) -- [TRAIN] RowParallelLinear / ColumnParallelLinear
// sections; a sum, never a mean ([TUT] §三).
//
// HBM-bound streaming kernel: each thread owns 8 consecutive elements, issues
// the 16-B loads of up to 8 partials back to back, then adds them in the fixed
// order 0..t-1 in fp32 (bit-reproducible), and writes one 16-B (bf16) or
// 2×16-B (fp32) store.  A scalar kernel covers the tail and unaligned inputs.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int RT = 256;

template <typename T>
struct Vec8;

template <>
struct Vec8<bf16> {
  u32x4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
  __device__ __forceinline__ void add_to(float (&acc)[8]) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += __uint_as_float(v[q] << 16);
      acc[2 * q + 1] += __uint_as_float(v[q] & 0xFFFF0000u);
    }
  }
};

template <>
struct Vec8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ void add_to(float (&acc)[8]) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q] += lo[q];
      acc[4 + q] += hi[q];
    }
  }
};

__device__ __forceinline__ void store8(bf16* p, const float (&acc)[8]) {
  bf16x8 o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = f2bf(acc[q]);
  *reinterpret_cast<bf16x8*>(p) = o;
}

__device__ __forceinline__ void store8(float* p, const float (&acc)[8]) {
  f32x4 lo, hi;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lo[q] = acc[q];
    hi[q] = acc[4 + q];
  }
  reinterpret_cast<f32x4*>(p)[0] = lo;
  reinterpret_cast<f32x4*>(p)[1] = hi;
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(RT) void reduce_vec8_kernel(const Tin* __restrict__ p, Tout* __restrict__ out,
                                                         int t, int64_t nvec, int64_t count) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * RT;
  for (int64_t v = static_cast<int64_t>(blockIdx.x) * RT + threadIdx.x; v < nvec; v += step) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const Tin* src = p + v * 8;
    for (int i0 = 0; i0 < t; i0 += 8) {
      Vec8<Tin> in[8];
      const int n = t - i0 < 8 ? t - i0 : 8;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) in[i].load(src + static_cast<int64_t>(i0 + i) * count);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) in[i].add_to(acc);
    }
    store8(out + v * 8, acc);
  }
}

template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (sizeof(T) == 2) return bf2f(*p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void st1(T* p, float v) {
  if constexpr (sizeof(T) == 2) *p = f2bf(v);
  else *p = v;
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(RT) void reduce_scalar_kernel(const Tin* __restrict__ p, Tout* __restrict__ out,
                                                           int t, int64_t begin, int64_t count) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * RT;
  for (int64_t e = begin + static_cast<int64_t>(blockIdx.x) * RT + threadIdx.x; e < count; e += step) {
    float acc = 0.f;
    for (int i = 0; i < t; ++i) acc += ld1(p + static_cast<int64_t>(i) * count + e);
    st1(out + e, acc);
  }
}

template <typename Tin, typename Tout>
hipError_t run(int t, int64_t count, const void* partials, void* out, hipStream_t stream) {
  const Tin* p = static_cast<const Tin*>(partials);
  Tout* o = static_cast<Tout*>(out);
  const bool aligned = (reinterpret_cast<uintptr_t>(p) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (count % 8 == 0);
  int64_t done = 0;
  if (aligned) {
    const int64_t nvec = count / 8;
    int64_t blocks = (nvec + RT - 1) / RT;
    if (blocks > 8192) blocks = 8192;
    if (blocks > 0) {
      hipLaunchKernelGGL((reduce_vec8_kernel<Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(RT), 0,
                         stream, p, o, t, nvec, count);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    done = nvec * 8;
  }
  if (done < count) {
    int64_t blocks = (count - done + RT - 1) / RT;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL((reduce_scalar_kernel<Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(RT), 0,
                       stream, p, o, t, done, count);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_reduce_partials(int in_dt, int out_dt, int t, int64_t count, const void* partials,
                                  void* out, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  if (in_dt == 1 && out_dt == 1) return run<bf16, bf16>(t, count, partials, out, stream);
  if (in_dt == 1 && out_dt == 0) return run<bf16, float>(t, count, partials, out, stream);
  if (in_dt == 0 && out_dt == 1) return run<float, bf16>(t, count, partials, out, stream);
  return run<float, float>(t, count, partials, out, stream);
}

}  // namespace tpmlp
