// GeLU(z) = z·Φ(z) and GeLU'(z) = Φ(z) + z·φ(z) for the bf16 GEMM epilogues,
// with no transcendental instruction.
//
// Φ(z) − ½ and GeLU'(z) − ½ are odd functions of z, so on |z| ≤ T each is
// z·P(z²) for a polynomial P.  P is a degree-9 near-minimax fit on [0, T],
// T = 4.5, written for this library (Lawson-reweighted least squares in a
// Chebyshev basis, then expanded to monomials in u = z² and rounded to fp32).
// Outside [−T, T] the argument is clamped to ±T:
//   * the Φ fit is pinned to reach 1 + 1e-5 at z = T (and −1e-5 at −T), and
//     the result is clamped to [0, 1], so Φ is exactly 1 for z ≥ T and exactly
//     0 for z ≤ −T, and GeLU is exactly z resp. 0 there;
//   * the GeLU' fit is pinned to GeLU'(T) at z = T.
// Evaluated in fp32 (Horner with fma), over all of ℝ:
//   |Φ̂ − Φ| ≤ 1.6e-5,  |GeLU_hat − GeLU| ≤ 7e-5,  |GeLU'_hat − GeLU'| ≤ 1.5e-4,
// against bf16's relative resolution of 2^-9 ≈ 2e-3 on the stored results.
// The coefficient lists below are parsed by the CPU test of these bounds:
// keep one `= { ... };` initialiser per list.
#pragma once

#include <hip/hip_runtime.h>

namespace tpmlp {

constexpr float kGeluPolyClamp = 4.5f;

// Φ(z) − ½ = z · Σ_k kPhiPoly[k] · u^k,  u = z², |z| ≤ 4.5
constexpr float kPhiPoly[10] = {
    3.988821805e-01f, -6.628771126e-02f, 9.771027602e-03f, -1.093266066e-03f, 9.082995530e-05f,
    -5.407767276e-06f, 2.187211550e-07f, -5.543902670e-09f, 7.614309877e-11f, -3.960302138e-13f};

// GeLU'(z) − ½ = z · Σ_k kGeluGradPoly[k] · u^k,  u = z², |z| ≤ 4.5
constexpr float kGeluGradPoly[10] = {
    7.976167202e-01f, -2.648935318e-01f, 5.857777223e-02f, -8.801988326e-03f, 9.372726781e-04f,
    -7.077334158e-05f, 3.685003776e-06f, -1.250099899e-07f, 2.473846905e-09f, -2.158200875e-11f};

template <int NC>
__device__ __forceinline__ float horner(const float (&c)[NC], float u) {
  float p = c[NC - 1];
#pragma unroll
  for (int k = NC - 2; k >= 0; --k) p = fmaf(p, u, c[k]);
  return p;
}

__device__ __forceinline__ float gelu_fast(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -kGeluPolyClamp, kGeluPolyClamp);
  const float phi = fmaf(zc, horner(kPhiPoly, zc * zc), 0.5f);
  return z * __builtin_amdgcn_fmed3f(phi, 0.0f, 1.0f);
}

__device__ __forceinline__ float gelu_grad_fast(float z) {
  const float zc = __builtin_amdgcn_fmed3f(z, -kGeluPolyClamp, kGeluPolyClamp);
  return fmaf(zc, horner(kGeluGradPoly, zc * zc), 0.5f);
}

}  // namespace tpmlp
