// out = Σ_{i<t} partials[i] (+ bias): the one-GPU stand-in for the
// tensor-parallel all-reduce after the row-parallel GEMM (forward) and of the
// column-parallel input gradient (backward) -- [TRAIN] RowParallelLinear /
// ColumnParallelLinear sections; a sum, never a mean ([TUT] §三).  The
// row-parallel layer's bias is not split: it is added once, after the sum
// ([TRAIN] RowParallelLinear).
//
// HBM-bound streaming kernel: each thread owns 8 consecutive elements, issues
// the 16-B loads of up to 8 partials back to back, then adds them in the fixed
// order 0..t-1 in fp32 (bit-reproducible), adds the bias, and writes one 16-B
// (bf16) or 2×16-B (fp32) store.  A scalar kernel covers the tail and
// unaligned inputs.  A thread's column advances by a fixed amount per
// grid-stride step, so the bias index needs one division per thread.
//
// Bias gradient db[i] = Σ_rows g[i] ([TRAIN] custom autograd matmul: the bias
// gradient is the upstream gradient summed over the tokens), in two fixed-order
// stages: per 128-row chunk column partials, then a sum over the chunks.  Both
// stages split their sums into 8 interleaved or consecutive parts to have
// enough loads in flight, and combine the parts in a fixed order.
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

// the 8 bias values at p (16-B aligned), widened; cached loads (reused)
__device__ __forceinline__ void bias8(const bf16* p, float (&b)[8]) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    b[2 * q] = __uint_as_float(u[q] << 16);
    b[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void bias8(const float* p, float (&b)[8]) {
  const f32x4 lo = reinterpret_cast<const f32x4*>(p)[0], hi = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    b[q] = lo[q];
    b[4 + q] = hi[q];
  }
}

// bias: NULL or [cols] of Tout; with a bias, cols % 8 == 0 (each vector lies
// in one row).  col tracks v·8 mod cols.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(RT) void reduce_vec8_kernel(const Tin* __restrict__ p, Tout* __restrict__ out,
                                                         int t, int64_t nvec, int64_t count,
                                                         const Tout* __restrict__ bias, int64_t cols) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * RT;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * RT + threadIdx.x;
  int64_t col = 0, dcol = 0;
  if (bias != nullptr) {
    col = (v0 * 8) % cols;
    dcol = (step * 8) % cols;
  }
  for (int64_t v = v0; v < nvec; v += step) {
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
    if (bias != nullptr) {
      float b[8];
      bias8(bias + col, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += b[q];
      col += dcol;
      if (col >= cols) col -= cols;
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

// 8 consecutive elements at p (16-B aligned), read once: nontemporal
template <typename T>
__device__ __forceinline__ void load8nt(const T* p, float (&w)[8]) {
  Vec8<T> v;
  v.load(p);
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = 0.f;
  v.add_to(w);
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(RT) void reduce_scalar_kernel(const Tin* __restrict__ p, Tout* __restrict__ out,
                                                           int t, int64_t begin, int64_t count,
                                                           const Tout* __restrict__ bias, int64_t cols) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * RT;
  const int64_t e0 = begin + static_cast<int64_t>(blockIdx.x) * RT + threadIdx.x;
  int64_t col = 0, dcol = 0;
  if (bias != nullptr) {
    col = e0 % cols;
    dcol = step % cols;
  }
  for (int64_t e = e0; e < count; e += step) {
    float acc = 0.f;
    for (int i = 0; i < t; ++i) acc += ld1(p + static_cast<int64_t>(i) * count + e);
    if (bias != nullptr) {
      acc += ld1(bias + col);
      col += dcol;
      if (col >= cols) col -= cols;
    }
    st1(out + e, acc);
  }
}

// ---------------------------------------------------------------- bias gradient
// Stage 1: block (x = chunk·ncb + column block, y = i) sums rows
// [chunk·BG_RC, +BG_RC) of g[i] for BG_CG column groups of W columns; thread (phase r, group c) adds rows
// r, r + BG_RP, ... in increasing order, then the BG_RP phase sums are added in
// phase order through LDS.  ws[i][chunk][cols] receives the chunk's sums.
constexpr int BG_RC = 128, BG_CG = 32, BG_RP = RT / BG_CG;

template <typename T, int W>
__global__ __launch_bounds__(RT) void bias_grad_partial_kernel(const T* __restrict__ g, float* __restrict__ ws,
                                                               int64_t rows, int64_t cols, int64_t nchunk,
                                                               int ncb) {
  __shared__ float red[BG_RP][BG_CG][W];
  const int c = threadIdx.x % BG_CG, r = threadIdx.x / BG_CG;
  const int64_t chunk = blockIdx.x / ncb, i = blockIdx.y;
  const int64_t col = (static_cast<int64_t>(blockIdx.x % ncb) * BG_CG + c) * W;
  const int64_t r0 = chunk * BG_RC, r1 = r0 + BG_RC < rows ? r0 + BG_RC : rows;
  const T* gi = g + i * rows * cols;
  float s[W];
#pragma unroll
  for (int k = 0; k < W; ++k) s[k] = 0.f;
  if (col < cols) {
    int64_t row = r0 + r;
    // groups of 4 rows: loads in flight together, added in row order
    for (; row + 3 * BG_RP < r1; row += 4 * BG_RP) {
      float w[4][W];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const T* q = gi + (row + u * BG_RP) * cols + col;
        if constexpr (W == 8) load8nt(q, w[u]);
        else w[u][0] = ld1(q);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < W; ++k) s[k] += w[u][k];
    }
    for (; row < r1; row += BG_RP) {
      const T* q = gi + row * cols + col;
      float w[W];
      if constexpr (W == 8) load8nt(q, w);
      else w[0] = ld1(q);
#pragma unroll
      for (int k = 0; k < W; ++k) s[k] += w[k];
    }
  }
#pragma unroll
  for (int k = 0; k < W; ++k) red[r][c][k] = s[k];
  __syncthreads();
  if (r == 0 && col < cols) {
    float* o = ws + (i * nchunk + chunk) * cols + col;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < BG_RP; ++q) a += red[q][c][k];
      o[k] = a;
    }
  }
}

// Stage 2: db[i][c] = Σ_chunk ws[i][chunk][c].  A block takes BG_CG of the
// t·cols outputs; thread (range g, column c) sums chunk range g of BG_RP
// consecutive ranges in increasing chunk order, then the range sums of each
// output are added in range order: a fixed order for any launch.
__global__ __launch_bounds__(RT) void bias_grad_final_kernel(const float* __restrict__ ws, float* __restrict__ db,
                                                             int64_t t, int64_t cols, int64_t nchunk) {
  __shared__ float part[BG_RP][BG_CG];
  const int c = threadIdx.x % BG_CG, g = threadIdx.x / BG_CG;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * BG_CG + c;
  const int64_t per = (nchunk + BG_RP - 1) / BG_RP;
  const int64_t k0 = g * per, k1 = k0 + per < nchunk ? k0 + per : nchunk;
  float s = 0.f;
  if (e < t * cols) {
    const int64_t i = e / cols, col = e - i * cols;
    const float* w = ws + i * nchunk * cols + col;
    int64_t k = k0;
    for (; k + 4 <= k1; k += 4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = w[(k + u) * cols];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; k < k1; ++k) s += w[k * cols];
  }
  part[g][c] = s;
  __syncthreads();
  if (g == 0 && e < t * cols) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < BG_RP; ++q) a += part[q][c];
    db[e] = a;
  }
}

__global__ __launch_bounds__(RT) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * RT + threadIdx.x;
  if (e < n) p[e] = 0.f;
}

template <typename T>
hipError_t run_bias_grad(int t, int64_t rows, int64_t cols, const void* g, float* db, float* ws,
                         hipStream_t stream) {
  if (rows == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((t * cols + RT - 1) / RT)), dim3(RT), 0,
                       stream, db, static_cast<int64_t>(t) * cols);
    return hipGetLastError();
  }
  const int64_t nchunk = bias_grad_chunks(rows);
  const T* gp = static_cast<const T*>(g);
  const bool vec = cols % 8 == 0 && reinterpret_cast<uintptr_t>(g) % 16 == 0;
  const int64_t w = vec ? 8 : 1;
  const int ncb = static_cast<int>((cols / w + BG_CG - 1) / BG_CG);
  const dim3 grid(static_cast<unsigned>(ncb * nchunk), static_cast<unsigned>(t));
  if (vec)
    hipLaunchKernelGGL((bias_grad_partial_kernel<T, 8>), grid, dim3(RT), 0, stream, gp, ws, rows, cols, nchunk,
                       ncb);
  else
    hipLaunchKernelGGL((bias_grad_partial_kernel<T, 1>), grid, dim3(RT), 0, stream, gp, ws, rows, cols, nchunk,
                       ncb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bias_grad_final_kernel, dim3(static_cast<unsigned>((t * cols + BG_CG - 1) / BG_CG)), dim3(RT),
                     0, stream, ws, db, static_cast<int64_t>(t), cols, nchunk);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t run(int t, int64_t count, const void* partials, void* out, const void* bias_v, int64_t cols,
               hipStream_t stream) {
  const Tin* p = static_cast<const Tin*>(partials);
  Tout* o = static_cast<Tout*>(out);
  const Tout* bias = static_cast<const Tout*>(bias_v);
  const bool aligned = (reinterpret_cast<uintptr_t>(p) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (count % 8 == 0) &&
                       (bias == nullptr || (cols % 8 == 0 && reinterpret_cast<uintptr_t>(bias) % 16 == 0));
  int64_t done = 0;
  if (aligned) {
    const int64_t nvec = count / 8;
    int64_t blocks = (nvec + RT - 1) / RT;
    if (blocks > 8192) blocks = 8192;
    if (blocks > 0) {
      hipLaunchKernelGGL((reduce_vec8_kernel<Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(RT), 0,
                         stream, p, o, t, nvec, count, bias, cols);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    done = nvec * 8;
  }
  if (done < count) {
    int64_t blocks = (count - done + RT - 1) / RT;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL((reduce_scalar_kernel<Tin, Tout>), dim3(static_cast<unsigned>(blocks)), dim3(RT), 0,
                       stream, p, o, t, done, count, bias, cols);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_reduce_partials(int in_dt, int out_dt, int t, int64_t count, const void* partials,
                                  void* out, const void* bias, int64_t cols, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  if (in_dt == 1 && out_dt == 1) return run<bf16, bf16>(t, count, partials, out, bias, cols, stream);
  if (in_dt == 1 && out_dt == 0) return run<bf16, float>(t, count, partials, out, bias, cols, stream);
  if (in_dt == 0 && out_dt == 1) return run<float, bf16>(t, count, partials, out, bias, cols, stream);
  return run<float, float>(t, count, partials, out, bias, cols, stream);
}

int64_t bias_grad_chunks(int64_t rows) { return rows <= 0 ? 0 : (rows + BG_RC - 1) / BG_RC; }

hipError_t launch_bias_grad_final(int t, int64_t rows, int64_t cols, float* db, const float* ws,
                                  hipStream_t stream) {
  if (t <= 0 || cols <= 0) return hipSuccess;
  if (rows <= 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((t * cols + RT - 1) / RT)), dim3(RT), 0, stream,
                       db, static_cast<int64_t>(t) * cols);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(bias_grad_final_kernel, dim3(static_cast<unsigned>((t * cols + BG_CG - 1) / BG_CG)), dim3(RT), 0,
                     stream, ws, db, static_cast<int64_t>(t), cols, bias_grad_chunks(rows));
  return hipGetLastError();
}

hipError_t launch_bias_grad(int dt, int t, int64_t rows, int64_t cols, const void* g, float* db, float* ws,
                            hipStream_t stream) {
  if (t <= 0 || cols <= 0) return hipSuccess;
  return dt == 1 ? run_bias_grad<bf16>(t, rows, cols, g, db, ws, stream)
                 : run_bias_grad<float>(t, rows, cols, g, db, ws, stream);
}

}  // namespace tpmlp
