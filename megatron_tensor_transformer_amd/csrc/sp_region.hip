// Sequence-parallel region around the MLP block ([SP] placement diagram and
// f/g operator table; [EFF] §3.5.1 backward chain; [TRAIN] LayerNorm and
// Dropout sections):
//   forward   U = LN(x) (row blocks of all t sequence shards = the AllGather),
//             out = x + dropout_p(Σ_i P_i + b)  (sum, then the row blocks are
//                                             the ReduceScatter's shards; the
//                                             optional bias b of the
//                                             row-parallel layer is added after
//                                             the reduction and fused with the
//                                             dropout and the residual add,
//                                             [EFF] §4.2)
//   backward  dS = g_out ⊙ mask / (1-p)      (the MLP's upstream gradient)
//             dx = g_out + LN'(Σ_i dU_i);  dγ = Σ_rows dU⊙x̂;  dβ = Σ_rows dU
//
// All kernels are HBM-bound and work on 8-element (16-B bf16) chunks; sums of
// the t partials load them in unconditional groups so the loads are in flight
// together, and add them in shard order.  For h ≤ 4096, LN forward gives each
// row one wave (at most 8 chunks per lane, in registers) and reduces with
// cross-lane shuffles, and LN backward works in 512-thread blocks (thread j
// owns chunk j of every row) with shuffles plus a fixed-order sum over the 8
// waves; each block walks a strided set of rows, so its dγ/dβ column partials
// stay in registers.  Wider rows loop over 4096-element pieces of the row (a
// block per row; LN backward first forms the two row means, then dx and the
// column partials per 4096-column slab).  The sums are deterministic:
// per-block partials in a fixed row order, then a fixed-order sum over blocks.
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
constexpr int LNB_THREADS = 512;  // LN backward block: 8 waves
constexpr int LNB_WAVES = LNB_THREADS / WAVE;
constexpr int LNB_MAX_BLOCKS = 512;  // LN backward grid (two blocks per CU), rows strided over it

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
    // one 32×32→64-bit product each (v_mad_u64_u32) instead of separate hi/lo
    const uint64_t p0 = static_cast<uint64_t>(M0) * c0, p1 = static_cast<uint64_t>(M1) * c2;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
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
// NT: a read-once streaming operand, loaded nontemporally so it does not
// displace reused data in the caches.
template <typename T, bool NT = true>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 u = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))
                       : *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(u[q] << 16);
      v[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
    }
  } else {
    const f32x4 lo = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p))
                        : reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 hi = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1)
                        : reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = lo[q];
      v[4 + q] = hi[q];
    }
  }
}

// v = Σ_{i<t} p[i·stride .. +7] in shard order.  Whole groups of 8, then 4,
// then single partials: each group's loads are unconditional, so they are
// issued back to back and waited for once.
template <typename T, int G>
__device__ __forceinline__ void add_group8(const T* p, int64_t stride, float (&v)[8]) {
  float w[G][8];
#pragma unroll
  for (int u = 0; u < G; ++u) load8(p + static_cast<int64_t>(u) * stride, w[u]);
#pragma unroll
  for (int u = 0; u < G; ++u)
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += w[u][k];
}

template <typename T>
__device__ __forceinline__ void sum_partials8(const T* p, int64_t stride, int t, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.f;
  int i = 0;
  for (; i + 8 <= t; i += 8) add_group8<T, 8>(p + static_cast<int64_t>(i) * stride, stride, v);
  if (i + 4 <= t) {
    add_group8<T, 4>(p + static_cast<int64_t>(i) * stride, stride, v);
    i += 4;
  }
  for (; i < t; ++i) add_group8<T, 1>(p + static_cast<int64_t>(i) * stride, stride, v);
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

// ------------------------------------------------------------------ raw 16-B loads
// Buffer loads whose offset may be past the buffer's range (then they read
// zeros and touch no memory), so every wave issues the same number of loads
// whether or not a row exists: the compiler's counted waits then let the next
// row's loads stay in flight while the current row is computed.
extern "C" __device__ i32x4 tpmlp_llvm_buffer_load_v4(i32x4 rsrc, int voffset, int soffset,
                                                      int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
constexpr uint32_t SP_OOB = 0x80000000u;  // past every range (operands are < 2^31 bytes)
constexpr int AUX_NT = 2;                 // nontemporal: read once

__device__ __forceinline__ i32x4 raw_load(i32x4 rsrc, uint32_t off) {
  return tpmlp_llvm_buffer_load_v4(rsrc, static_cast<int>(off), 0, AUX_NT);
}

// 8 bf16 values held as one 16-B word -> fp32
__device__ __forceinline__ void raw_to_f(i32x4 r, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u = static_cast<uint32_t>(r[q]);
    v[2 * q] = __uint_as_float(u << 16);
    v[2 * q + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
}

// ------------------------------------------------------------------ LN forward
// bf16, h ≤ 4096: a wave walks rows r, r + W, ... (W waves in the grid); the
// next row's loads are issued before the current row is reduced and written,
// so each wave keeps a row in flight while it computes.  The γ and β chunks of
// the output are loaded before the next row's prefetch, so waiting for them
// leaves the prefetch in flight.
__global__ __launch_bounds__(SP_THREADS) void ln_fwd_pipe_kernel(SpProblem p) {
  constexpr int MAXC = 8;
  const int lane = threadIdx.x & 63;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (SP_THREADS / WAVE);
  int64_t row = static_cast<int64_t>(blockIdx.x) * (SP_THREADS / WAVE) + (threadIdx.x >> 6);
  if (row >= p.s) return;
  const int hc = static_cast<int>(p.h / 8);
  const float inv_h = 1.0f / static_cast<float>(p.h);
  const i32x4 rx = make_rsrc(p.x, static_cast<uint32_t>(p.s * p.h * 2));
  const i32x4 rg = make_rsrc(p.gamma, static_cast<uint32_t>(p.h * 2));
  const i32x4 rb = make_rsrc(p.beta, static_cast<uint32_t>(p.h * 2));
  i32x4 nxt[MAXC];
  auto issue = [&](int64_t r) {
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      const int c = lane + WAVE * k;
      nxt[k] = raw_load(rx, r < p.s && c < hc ? static_cast<uint32_t>((r * p.h + c * 8) * 2) : SP_OOB);
    }
  };
  issue(row);
  for (;;) {
    float v[MAXC][8];
#pragma unroll
    for (int k = 0; k < MAXC; ++k) raw_to_f(nxt[k], v[k]);  // chunks past h read as zeros
    i32x4 g[MAXC], b[MAXC];
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      const int c = lane + WAVE * k;
      const uint32_t off = c < hc ? static_cast<uint32_t>(c * 16) : SP_OOB;
      g[k] = tpmlp_llvm_buffer_load_v4(rg, static_cast<int>(off), 0, 0);
      b[k] = tpmlp_llvm_buffer_load_v4(rb, static_cast<int>(off), 0, 0);
    }
    issue(row + nw);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += v[k][e];
    sum = wave_sum(sum);
    const float mean = sum * inv_h;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      if (lane + WAVE * k < hc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[k][e] - mean;
          q += d * d;
        }
      }
    }
    q = wave_sum(q);
    const float rstd = 1.0f / sqrtf(q * inv_h + p.eps);
    bf16* yr = static_cast<bf16*>(p.ln_out) + row * p.h;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
      const int c = lane + WAVE * k;
      if (c < hc) {
        float gf[8], bf[8], o[8];
        raw_to_f(g[k], gf);
        raw_to_f(b[k], bf);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf((v[k][e] - mean) * rstd, gf[e], bf[e]);
        store8(yr + c * 8, o);
      }
    }
    if (lane == 0) {
      p.mean[row] = mean;
      p.rstd[row] = rstd;
    }
    row += nw;
    if (row >= p.s) break;
  }
  wait_vmcnt<0>();  // the last (empty) prefetch
}

// A 512-thread block normalises rows 2b and 2b+1; thread j owns chunk j of
// each (h ≤ 4096).  Two passes over the registers (mean, then the biased
// variance of x - mean), each a wave sum combined over the 8 waves in a fixed
// order through LDS.
__device__ __forceinline__ void block_sum2(float (&v)[2], float (*red)[2], int lane, int wave) {
  v[0] = wave_sum(v[0]);
  v[1] = wave_sum(v[1]);
  if (lane == 0) {
    red[wave][0] = v[0];
    red[wave][1] = v[1];
  }
  __syncthreads();
  v[0] = v[1] = 0.f;
#pragma unroll
  for (int w = 0; w < LNB_WAVES; ++w) {
    v[0] += red[w][0];
    v[1] += red[w][1];
  }
}

// LN forward: one wave per row (h ≤ 4096: at most 8 16-B chunks per lane, all
// loaded before the first use, so a wave keeps 8 KB in flight); mean and
// variance are wave sums in a fixed lane order (butterfly), no LDS or barrier.
template <typename T>
__global__ __launch_bounds__(SP_THREADS) void ln_fwd_kernel(SpProblem p) {
  constexpr int MAXC = 8;  // chunks per lane for h ≤ 4096
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (SP_THREADS / WAVE) + (threadIdx.x >> 6);
  if (row >= p.s) return;
  const int hc = p.h / 8;
  const T* xr = static_cast<const T*>(p.x) + row * p.h;
  float v[MAXC][8];
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = lane + WAVE * k;
    if (c < hc) {
      load8(xr + c * 8, v[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
    }
  }
  const float inv_h = 1.0f / static_cast<float>(p.h);
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < MAXC; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[k][e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, WAVE);
  const float mean = sum * inv_h;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    if (lane + WAVE * k < hc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[k][e] - mean;
        q += d * d;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) q += __shfl_xor(q, o, WAVE);
  const float rstd = 1.0f / sqrtf(q * inv_h + p.eps);
  T* yr = static_cast<T*>(p.ln_out) + row * p.h;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = lane + WAVE * k;
    if (c < hc) {
      float g[8], b[8], o[8];
      load8<T, false>(static_cast<const T*>(p.gamma) + c * 8, g);
      load8<T, false>(static_cast<const T*>(p.beta) + c * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf((v[k][e] - mean) * rstd, g[e], b[e]);
      store8(yr + c * 8, o);
    }
  }
  if (lane == 0) {
    p.mean[row] = mean;
    p.rstd[row] = rstd;
  }
}

// ------------------------------------------------------------------ wide rows (h > 4096)
// Rows wider than 8 chunks per lane of a wave (h > 4096) take a 512-thread
// block per row, which loops over the row in 4096-element pieces (thread j
// owns chunks j, j + 512, ...), re-reading the row from the cache in each
// pass instead of holding it in registers.
constexpr int LNW_THREADS = 512, LNW_WAVES = LNW_THREADS / WAVE;
constexpr int64_t LN_FAST_MAX_H = 4096;

// Sum over the block in a fixed order: each wave's butterfly, then the waves'
// sums in wave order.  Every thread gets the result; `red` may be reused
// right after (the trailing barrier).
__device__ __forceinline__ float block_sum_fixed(float v, float* red, int lane, int wave) {
  v = wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < LNW_WAVES; ++w) s += red[w];
  __syncthreads();
  return s;
}

template <typename T>
__global__ __launch_bounds__(LNW_THREADS) void ln_fwd_wide_kernel(SpProblem p) {
  __shared__ float red[LNW_WAVES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int64_t hc = p.h / 8;
  const float inv_h = 1.0f / static_cast<float>(p.h);
  const T* xr = static_cast<const T*>(p.x) + row * p.h;
  float sum = 0.f;
  for (int64_t c = threadIdx.x; c < hc; c += LNW_THREADS) {
    float v[8];
    load8<T, false>(xr + c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += v[e];
  }
  const float mean = block_sum_fixed(sum, red, lane, wave) * inv_h;
  float q = 0.f;
  for (int64_t c = threadIdx.x; c < hc; c += LNW_THREADS) {
    float v[8];
    load8<T, false>(xr + c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[e] - mean;
      q += d * d;
    }
  }
  const float rstd = 1.0f / sqrtf(block_sum_fixed(q, red, lane, wave) * inv_h + p.eps);
  T* yr = static_cast<T*>(p.ln_out) + row * p.h;
  for (int64_t c = threadIdx.x; c < hc; c += LNW_THREADS) {
    float v[8], g[8], b[8], o[8];
    load8<T, false>(xr + c * 8, v);
    load8<T, false>(static_cast<const T*>(p.gamma) + c * 8, g);
    load8<T, false>(static_cast<const T*>(p.beta) + c * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf((v[e] - mean) * rstd, g[e], b[e]);
    store8(yr + c * 8, o);
  }
  if (threadIdx.x == 0) {
    p.mean[row] = mean;
    p.rstd[row] = rstd;
  }
}

// LN backward, wide rows, pass 1: the two row means of the input gradient,
// m1 = mean(dU⊙γ) and m2 = mean(dU⊙γ⊙x̂) with dU = Σ_i dU_i (shard order),
// to rowstats[row][0..1].
template <typename T>
__global__ __launch_bounds__(LNW_THREADS) void ln_bwd_rowstats_kernel(SpProblem p, float* __restrict__ rowstats) {
  __shared__ float red[LNW_WAVES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int64_t hc = p.h / 8, count = p.s * p.h;
  const float mu = p.mean[row], rs = p.rstd[row];
  float s1 = 0.f, s2 = 0.f;
  for (int64_t c = threadIdx.x; c < hc; c += LNW_THREADS) {
    const int64_t off = row * p.h + c * 8;
    float du[8], xh[8], gq[8];
    load8<T, false>(static_cast<const T*>(p.x) + off, xh);
    load8<T, false>(static_cast<const T*>(p.gamma) + c * 8, gq);
    sum_partials8(static_cast<const T*>(p.dU_partials) + off, count, p.t, du);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float gt = du[k] * gq[k];
      s1 += gt;
      s2 += gt * ((xh[k] - mu) * rs);
    }
  }
  const float inv_h = 1.0f / static_cast<float>(p.h);
  s1 = block_sum_fixed(s1, red, lane, wave);
  s2 = block_sum_fixed(s2, red, lane, wave);
  if (threadIdx.x == 0) {
    rowstats[2 * row] = s1 * inv_h;
    rowstats[2 * row + 1] = s2 * inv_h;
  }
}

// LN backward, wide rows, pass 2: block (b, slab) owns columns
// [4096·slab, 4096·slab + 4096) (thread j chunk 4096·slab/8 + j) of rows b,
// b + nb, ...; dx = g_out + rstd·(dU⊙γ − m1 − x̂·m2) with dU summed again in
// the same order as pass 1, and the thread's column partials of dU⊙x̂ and dU
// go to ws[b][0|1][h].
template <typename T>
__global__ __launch_bounds__(LNW_THREADS) void ln_bwd_wide_kernel(SpProblem p, const float* __restrict__ rowstats) {
  const int64_t c = static_cast<int64_t>(blockIdx.y) * LNW_THREADS + threadIdx.x;
  const bool mine = c < p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t nb = gridDim.x;
  float gq[8], dg[8], db[8];
  if (mine) load8<T, false>(static_cast<const T*>(p.gamma) + c * 8, gq);
#pragma unroll
  for (int k = 0; k < 8; ++k) dg[k] = db[k] = 0.f;
  if (mine) {
    for (int64_t row = blockIdx.x; row < p.s; row += nb) {
      const int64_t off = row * p.h + c * 8;
      const float mu = p.mean[row], rs = p.rstd[row];
      const float m1 = rowstats[2 * row], m2 = rowstats[2 * row + 1];
      float du[8], xh[8], go[8], o[8];
      load8(static_cast<const T*>(p.x) + off, xh);
      load8(static_cast<const T*>(p.g_out) + off, go);
      sum_partials8(static_cast<const T*>(p.dU_partials) + off, count, p.t, du);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xh[k] = (xh[k] - mu) * rs;
        o[k] = go[k] + rs * (du[k] * gq[k] - m1 - xh[k] * m2);
        dg[k] += du[k] * xh[k];
        db[k] += du[k];
      }
      store8(static_cast<T*>(p.dx) + off, o);
    }
    float* ws = p.ws + static_cast<int64_t>(blockIdx.x) * 2 * p.h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ws[c * 8 + k] = dg[k];
      ws[p.h + c * 8 + k] = db[k];
    }
  }
}

// ------------------------------------------------------------------ dropout + residual
// phase 1: out = x + keep·scale·(Σ_i P_i + b) ;  phase 2: dS = g_out·keep·scale
// With a bias, a thread's column chunk advances by a fixed amount per
// grid-stride step (h % 8 == 0, so a chunk lies in one row).
template <typename T, bool FWD>
__global__ __launch_bounds__(SP_THREADS) void dropres_kernel(SpProblem p) {
  const int64_t nchunk = p.s * p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t step = static_cast<int64_t>(gridDim.x) * SP_THREADS;
  const int64_t ch0 = static_cast<int64_t>(blockIdx.x) * SP_THREADS + threadIdx.x;
  const T* bias = FWD ? static_cast<const T*>(p.bias) : nullptr;
  const int64_t hc = p.h / 8;
  int64_t cc = 0, dcc = 0;
  if (bias != nullptr) {
    cc = ch0 % hc;
    dcc = step % hc;
  }
  for (int64_t ch = ch0; ch < nchunk; ch += step) {
    const int64_t e = ch * 8;  // local element index; rows are contiguous
    float v[8];
    if constexpr (FWD) {
      float xr[8];
      load8(static_cast<const T*>(p.x) + e, xr);  // in flight with the partials
      sum_partials8(static_cast<const T*>(p.partials) + e, count, p.t, v);
      if (bias != nullptr) {
        float b[8];
        load8<T, false>(bias + cc * 8, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] += b[k];
        cc += dcc;
        if (cc >= hc) cc -= hc;
      }
      const uint32_t keep = keep8(static_cast<uint64_t>(p.row0 * p.h + e), p.seed, p.drop_threshold);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = xr[k] + (((keep >> k) & 1u) ? v[k] * p.keep_scale : 0.0f);
      store8(static_cast<T*>(p.out) + e, v);
    } else {
      load8(static_cast<const T*>(p.g_out) + e, v);
      const uint32_t keep = keep8(static_cast<uint64_t>(p.row0 * p.h + e), p.seed, p.drop_threshold);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = ((keep >> k) & 1u) ? v[k] * p.keep_scale : 0.0f;
      store8(static_cast<T*>(p.dS) + e, v);
    }
  }
}

// Forward, bf16, t = 8 partials: the loads of x and the partials are issued
// first and the chunk's Philox blocks computed while they are in flight; the
// sum of the partials is then formed in shard order as in dropres_kernel, so
// the results are the same bit for bit.
__global__ __launch_bounds__(SP_THREADS) void dropres_fwd8_kernel(SpProblem p) {
  constexpr int T8 = 8;
  const int64_t nchunk = p.s * p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t step = static_cast<int64_t>(gridDim.x) * SP_THREADS;
  const int64_t ch0 = static_cast<int64_t>(blockIdx.x) * SP_THREADS + threadIdx.x;
  const bf16* bias = static_cast<const bf16*>(p.bias);
  const int64_t hc = p.h / 8;
  int64_t cc = 0, dcc = 0;
  if (bias != nullptr) {
    cc = ch0 % hc;
    dcc = step % hc;
  }
  const i32x4 rx = make_rsrc(p.x, static_cast<uint32_t>(count * 2));
  const i32x4 rp = make_rsrc(p.partials, static_cast<uint32_t>(T8 * count * 2));
  for (int64_t ch = ch0; ch < nchunk; ch += step) {
    const int64_t e = ch * 8;
    const uint32_t off = static_cast<uint32_t>(e * 2);
    const i32x4 xin = raw_load(rx, off);
    i32x4 pr[T8];
#pragma unroll
    for (int i = 0; i < T8; ++i) pr[i] = raw_load(rp, off + static_cast<uint32_t>(i * count * 2));
    // keep the loads ahead of the Philox arithmetic and the arithmetic ahead
    // of the first wait for their data (the scheduler would otherwise start
    // the sum first and leave the arithmetic for after the loads)
    __builtin_amdgcn_sched_barrier(0);
    uint32_t keep = keep8(static_cast<uint64_t>(p.row0 * p.h + e), p.seed, p.drop_threshold);
    asm volatile("" : "+v"(keep));  // materialised here, not sunk to its later use
    __builtin_amdgcn_sched_barrier(0);
    float v[8], xr[8];
    raw_to_f(xin, xr);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
#pragma unroll
    for (int i = 0; i < T8; ++i) {
      float w[8];
      raw_to_f(pr[i], w);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += w[k];
    }
    if (bias != nullptr) {
      float b[8];
      load8<bf16, false>(bias + cc * 8, b);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += b[k];
      cc += dcc;
      if (cc >= hc) cc -= hc;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xr[k] + (((keep >> k) & 1u) ? v[k] * p.keep_scale : 0.0f);
    store8(static_cast<bf16*>(p.out) + e, v);
  }
}

// ------------------------------------------------------------------ LN backward
// bf16, t = 8 partials, h ≤ 4096: ln_bwd_kernel with the next row's loads (x,
// g_out and the 8 partials) issued before the current row is reduced across
// the block and written, so a block keeps a row in flight while it computes.
// Same arithmetic in the same order as ln_bwd_kernel.
__global__ __launch_bounds__(LNB_THREADS, 2) void ln_bwd_pipe_kernel(SpProblem p) {
  constexpr int T8 = 8;
  __shared__ float red[2][LNB_WAVES][2];  // [row parity][wave][s1, s2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = threadIdx.x;
  const bool mine = c < p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t nb = gridDim.x;
  const float inv_h = 1.0f / static_cast<float>(p.h);
  const i32x4 rx = make_rsrc(p.x, static_cast<uint32_t>(count * 2));
  const i32x4 rg = make_rsrc(p.g_out, static_cast<uint32_t>(count * 2));
  const i32x4 rp = make_rsrc(p.dU_partials, static_cast<uint32_t>(T8 * count * 2));

  float gq[8], dg[8], db[8];
  if (mine) load8<bf16, false>(static_cast<const bf16*>(p.gamma) + c * 8, gq);
#pragma unroll
  for (int k = 0; k < 8; ++k) dg[k] = db[k] = 0.f;

  i32x4 nx, ng, np[T8];
  auto issue = [&](int64_t r) {
    const uint32_t off = r < p.s && mine ? static_cast<uint32_t>((r * p.h + c * 8) * 2) : SP_OOB;
    nx = raw_load(rx, off);
    ng = raw_load(rg, off);
#pragma unroll
    for (int i = 0; i < T8; ++i)
      np[i] = raw_load(rp, off == SP_OOB ? SP_OOB : off + static_cast<uint32_t>(i * count * 2));
  };
  int64_t row = blockIdx.x;
  issue(row);
  for (int par = 0;; par ^= 1) {
    float du[8], xh[8], go[8];
    raw_to_f(nx, xh);
    raw_to_f(ng, go);
#pragma unroll
    for (int k = 0; k < 8; ++k) du[k] = 0.f;
#pragma unroll
    for (int i = 0; i < T8; ++i) {
      float w[8];
      raw_to_f(np[i], w);
#pragma unroll
      for (int k = 0; k < 8; ++k) du[k] += w[k];
    }
    const float mu = p.mean[row], rs = p.rstd[row];
    issue(row + nb);
    float sm[2] = {0.f, 0.f};
    if (mine) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xh[k] = (xh[k] - mu) * rs;
        const float gt = du[k] * gq[k];
        sm[0] += gt;
        sm[1] += gt * xh[k];
        dg[k] += du[k] * xh[k];
        db[k] += du[k];
      }
    }
    sm[0] = wave_sum(sm[0]);
    sm[1] = wave_sum(sm[1]);
    if (lane == 0) {
      red[par][wave][0] = sm[0];
      red[par][wave][1] = sm[1];
    }
    __syncthreads();
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int w = 0; w < LNB_WAVES; ++w) {
      m1 += red[par][w][0];
      m2 += red[par][w][1];
    }
    // red[par] is rewritten two rows on, after the next barrier
    m1 *= inv_h;
    m2 *= inv_h;
    if (mine) {
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = go[k] + rs * (du[k] * gq[k] - m1 - xh[k] * m2);
      store8(static_cast<bf16*>(p.dx) + row * p.h + c * 8, o);
    }
    row += nb;
    if (row >= p.s) break;
  }
  wait_vmcnt<0>();  // the last (empty) prefetch
  const int64_t h = p.h;
  if (mine) {
    float* ws = p.ws + static_cast<int64_t>(blockIdx.x) * 2 * h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ws[c * 8 + k] = dg[k];
      ws[h + c * 8 + k] = db[k];
    }
  }
}

// Block b handles rows b, b + nb, b + 2·nb, ... (nb = gridDim.x); thread j
// owns chunk j of every row (h ≤ 4096).  Per row: dU = Σ_i dU_i,
// x̂ = (x-μ)·rstd, g̃ = dU⊙γ, dx = g_out + rstd·(g̃ - mean(g̃) - x̂·mean(g̃⊙x̂));
// the two row means are wave sums combined over the 8 waves in a fixed order
// through LDS.  The thread's column partials of dU⊙x̂ and dU go to
// ws[b][0|1][h] at the end.  Two blocks share a CU, so one's loads are in
// flight while the other computes.
template <typename T>
__global__ __launch_bounds__(LNB_THREADS, 2) void ln_bwd_kernel(SpProblem p) {
  __shared__ float red[2][LNB_WAVES][2];  // [row parity][wave][s1, s2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = threadIdx.x;
  const bool mine = c < p.h / 8;
  const int64_t count = p.s * p.h;
  const int64_t nb = gridDim.x;
  const float inv_h = 1.0f / static_cast<float>(p.h);

  float gq[8], dg[8], db[8];
  if (mine) load8<T, false>(static_cast<const T*>(p.gamma) + c * 8, gq);
#pragma unroll
  for (int k = 0; k < 8; ++k) dg[k] = db[k] = 0.f;

  int par = 0;
  for (int64_t row = blockIdx.x; row < p.s; row += nb, par ^= 1) {
    const int64_t off = row * p.h + c * 8;
    float du[8], xh[8], go[8];
    float sm[2] = {0.f, 0.f};
    const float mu = p.mean[row], rs = p.rstd[row];
    if (mine) {
      load8(static_cast<const T*>(p.x) + off, xh);
      load8(static_cast<const T*>(p.g_out) + off, go);
      sum_partials8(static_cast<const T*>(p.dU_partials) + off, count, p.t, du);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xh[k] = (xh[k] - mu) * rs;
        const float gt = du[k] * gq[k];
        sm[0] += gt;
        sm[1] += gt * xh[k];
        dg[k] += du[k] * xh[k];
        db[k] += du[k];
      }
    }
    sm[0] = wave_sum(sm[0]);
    sm[1] = wave_sum(sm[1]);
    if (lane == 0) {
      red[par][wave][0] = sm[0];
      red[par][wave][1] = sm[1];
    }
    __syncthreads();
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int w = 0; w < LNB_WAVES; ++w) {
      m1 += red[par][w][0];
      m2 += red[par][w][1];
    }
    // red[par] is rewritten two rows on, after the next barrier: no second
    // barrier is needed here.
    m1 *= inv_h;
    m2 *= inv_h;
    if (mine) {
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = go[k] + rs * (du[k] * gq[k] - m1 - xh[k] * m2);
      store8(static_cast<T*>(p.dx) + off, o);
    }
  }
  const int64_t h = p.h;
  if (mine) {
    float* ws = p.ws + static_cast<int64_t>(blockIdx.x) * 2 * h;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ws[c * 8 + k] = dg[k];
      ws[h + c * 8 + k] = db[k];
    }
  }
}

// dγ[j] = Σ_b ws[b][0][j], dβ[j] = Σ_b ws[b][1][j] over the nblk LN-backward
// blocks.  A 256-thread block takes 32 of the 2h columns; thread (g, c) sums
// block range g of 8 consecutive ranges in increasing b, then the 8 range sums
// of each column are added in range order: a fixed order for any launch.
constexpr int CS_COLS = 32, CS_GROUPS = SP_THREADS / CS_COLS;
__global__ __launch_bounds__(SP_THREADS) void colsum_kernel(const float* __restrict__ ws, int64_t nblk,
                                                            int64_t h, float* __restrict__ dgamma,
                                                            float* __restrict__ dbeta) {
  __shared__ float part[CS_GROUPS][CS_COLS];
  const int c = threadIdx.x % CS_COLS, g = threadIdx.x / CS_COLS;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * CS_COLS + c;
  const int64_t per = (nblk + CS_GROUPS - 1) / CS_GROUPS;
  const int64_t b0 = g * per, b1 = b0 + per < nblk ? b0 + per : nblk;
  float s = 0.f;
  if (j < 2 * h) {
    int64_t b = b0;
    for (; b + 8 <= b1; b += 8) {
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = ws[(b + u) * 2 * h + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += w[u];
    }
    for (; b < b1; ++b) s += ws[b * 2 * h + j];
  }
  part[g][c] = s;
  __syncthreads();
  if (g == 0 && j < 2 * h) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < CS_GROUPS; ++k) t += part[k][c];
    if (j < h) dgamma[j] = t;
    else dbeta[j - h] = t;
  }
}

template <typename T>
hipError_t launch_dt(const SpProblem& p, hipStream_t stream) {
  const bool wide = p.h > LN_FAST_MAX_H;
  switch (p.phase) {
    case 0: {
      if (wide) {
        hipLaunchKernelGGL((ln_fwd_wide_kernel<T>), dim3(static_cast<unsigned>(p.s)), dim3(LNW_THREADS), 0,
                           stream, p);
        return hipGetLastError();
      }
      if constexpr (sizeof(T) == 2) {
        // about two rows per wave, at most 2048 waves (8 per CU)
        const int64_t waves = (p.s + 1) / 2 < 2048 ? (p.s + 1) / 2 : 2048;
        const int64_t blocks = (waves + SP_THREADS / WAVE - 1) / (SP_THREADS / WAVE);
        hipLaunchKernelGGL(ln_fwd_pipe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0, stream, p);
        return hipGetLastError();
      }
      const int64_t blocks = (p.s + SP_THREADS / WAVE - 1) / (SP_THREADS / WAVE);  // one wave per row
      hipLaunchKernelGGL((ln_fwd_kernel<T>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0, stream,
                         p);
      return hipGetLastError();
    }
    case 1:
    case 2: {
      const int64_t nchunk = p.s * p.h / 8;
      int64_t blocks = (nchunk + SP_THREADS - 1) / SP_THREADS;
      if (blocks > 16384) blocks = 16384;
      if (sizeof(T) == 2 && p.phase == 1 && p.t == 8) {
        // (the backward's dropout kernel is bound by the Philox arithmetic:
        // issuing its one load ahead of it gained nothing, so it keeps the
        // plain form)
        hipLaunchKernelGGL(dropres_fwd8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0, stream, p);
      } else if (p.phase == 1)
        hipLaunchKernelGGL((dropres_kernel<T, true>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((dropres_kernel<T, false>), dim3(static_cast<unsigned>(blocks)), dim3(SP_THREADS),
                           0, stream, p);
      return hipGetLastError();
    }
    default: {
      const int64_t nblk = sp_ln_bwd_row_blocks(p.s, p.h);
      hipError_t e;
      if (wide) {
        // the row means first (rowstats after the per-block partials in ws),
        // then dx and the column partials in 4096-column slabs
        float* rowstats = p.ws + nblk * 2 * p.h;
        hipLaunchKernelGGL((ln_bwd_rowstats_kernel<T>), dim3(static_cast<unsigned>(p.s)), dim3(LNW_THREADS), 0,
                           stream, p, rowstats);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t slabs = (p.h / 8 + LNW_THREADS - 1) / LNW_THREADS;
        hipLaunchKernelGGL((ln_bwd_wide_kernel<T>), dim3(static_cast<unsigned>(nblk), static_cast<unsigned>(slabs)),
                           dim3(LNW_THREADS), 0, stream, p, static_cast<const float*>(rowstats));
      } else if (sizeof(T) == 2 && p.t == 8) {
        hipLaunchKernelGGL(ln_bwd_pipe_kernel, dim3(static_cast<unsigned>(nblk)), dim3(LNB_THREADS), 0, stream, p);
      } else {
        // one chunk of each row per thread
        hipLaunchKernelGGL((ln_bwd_kernel<T>), dim3(static_cast<unsigned>(nblk)), dim3(LNB_THREADS), 0,
                           stream, p);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t cb = (2 * p.h + CS_COLS - 1) / CS_COLS;
      hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>(cb)), dim3(SP_THREADS), 0, stream, p.ws,
                         nblk, p.h, p.dgamma, p.dbeta);
      return hipGetLastError();
    }
  }
}

}  // namespace

int64_t sp_ln_bwd_row_blocks(int64_t s, int64_t h) {
  // wide rows: the 4096-column slabs share the grid of about LNB_MAX_BLOCKS
  const int64_t slabs = h > LN_FAST_MAX_H ? (h / 8 + LNW_THREADS - 1) / LNW_THREADS : 1;
  const int64_t cap = (LNB_MAX_BLOCKS + slabs - 1) / slabs;
  return s < cap ? s : cap;
}

int64_t sp_workspace_floats(int64_t s, int64_t h) {
  // per row block: the column partials of dU⊙x̂ and dU; wide rows also keep
  // the two row means of every row
  return sp_ln_bwd_row_blocks(s, h) * 2 * h + (h > LN_FAST_MAX_H ? 2 * s : 0);
}

hipError_t launch_sp(const SpProblem& p, hipStream_t stream) {
  if (p.s <= 0) return hipSuccess;
  if (p.dt == 1) return launch_dt<bf16>(p, stream);
  return launch_dt<float>(p, stream);
}

}  // namespace tpmlp
