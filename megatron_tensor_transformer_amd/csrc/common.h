// Shared device helpers for the gfx950 kernels of the TP-MLP shard library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gelu_poly.h"  // GeLU / GeLU' of the bf16 epilogues

namespace tpmlp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TPMLP_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Buffer resources.  A raw buffer descriptor (stride 0) bounds every access by
// num_records bytes; an access whose offset is past the end returns zeros,
// which is how partial tiles at the matrix edges are zero-filled.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int>(static_cast<uint32_t>(p));
  r[1] = static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xFFFFu);  // stride 0
  r[2] = static_cast<int>(num_bytes);
  r[3] = 0x00020000;  // gfx9 data-format word for raw dword access
  return r;
}

// 16-byte load from a buffer straight into LDS.  Lane L of the wave writes
// bytes [16L, 16L+16) after the wave-uniform LDS address `lds`.
extern "C" __device__ void tpmlp_llvm_buffer_load_lds(i32x4 rsrc, TPMLP_LDS void* lds, int size,
                                                      int voffset, int soffset, int offset,
                                                      int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, TPMLP_LDS void* lds, uint32_t voff) {
  tpmlp_llvm_buffer_load_lds(rsrc, lds, 16, static_cast<int>(voff), 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

__device__ __forceinline__ void block_barrier() { __builtin_amdgcn_s_barrier(); }

// fp32 path: the device library's erf / exp, for ≤1e-5 parity in fp32.
__device__ __forceinline__ float gelu_precise(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_precise(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
         z * 0.39894228040143268f * expf(-0.5f * z * z);
}

// ---------------------------------------------------------------------------
// bf16 <-> f32.  The conversion to bf16 rounds to nearest even.
__device__ __forceinline__ float bf2f(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ bf16 f2bf(float v) { return static_cast<bf16>(v); }

}  // namespace tpmlp
