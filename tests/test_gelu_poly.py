"""Error bounds of the transcendental-free GeLU / GeLU' used by the bf16 GEMM
epilogues, checked on the CPU against scipy's erf.

The coefficients are read from the kernel header and evaluated the way the
kernel does (clamp to ±4.5, Horner in u = z² with fp32 fma, Φ clamped to
[0, 1]); fp32 fma is emulated by an exact fp64 product-sum rounded once to
fp32, which is exact-to-one-rounding as the hardware's fma is.
"""

import os
import re

import numpy as np
from scipy.special import erf

from conftest import ROOT

HEADER = os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc", "gelu_poly.h")


def coefficients(name):
    text = open(HEADER).read()
    m = re.search(name + r"\[\d+\]\s*=\s*\{(.*?)\};", text, flags=re.S)
    assert m, name
    return [np.float32(float(v.strip().rstrip("f"))) for v in m.group(1).split(",") if v.strip()]


def clamp_value():
    m = re.search(r"kGeluPolyClamp\s*=\s*([0-9.]+)f", open(HEADER).read())
    return np.float32(float(m.group(1)))


def fma32(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def poly_odd_half(coef, z):
    T = clamp_value()
    zc = np.clip(z, -T, T).astype(np.float32)
    u = (zc * zc).astype(np.float32)
    p = np.full_like(u, coef[-1])
    for c in coef[-2::-1]:
        p = fma32(p, u, np.full_like(u, c))
    return fma32(zc, p, np.full_like(u, np.float32(0.5)))


def phi_hat(z):
    return np.clip(poly_odd_half(coefficients("kPhiPoly"), z), 0, 1)


def gelu_hat(z):
    return (z * phi_hat(z)).astype(np.float32)


def gelu_grad_hat(z):
    return poly_odd_half(coefficients("kGeluGradPoly"), z)


def Phi(z):
    return 0.5 * (1.0 + erf(z / np.sqrt(2.0)))


def gelu_grad(z):
    return Phi(z) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


GRID = np.concatenate([np.linspace(-9.0, 9.0, 720001, dtype=np.float32),
                       np.array([-1e30, -1e4, -100.0, -4.5, 0.0, 4.5, 100.0, 1e4, 1e30], dtype=np.float32)])


def test_phi_error_bound():
    z = GRID.astype(np.float64)
    assert np.abs(phi_hat(GRID) - Phi(z)).max() <= 1.6e-5


def test_gelu_error_bound_everywhere():
    z = GRID.astype(np.float64)
    err = np.abs(gelu_hat(GRID).astype(np.float64) - z * Phi(z))
    # relative to |z| beyond the clamp (fp32 rounding of z·1), absolute inside
    assert err[np.abs(z) <= 9].max() <= 7e-5
    assert np.all(err <= 7e-5 + 1e-7 * np.abs(z))


def test_tails_are_exact():
    T = float(clamp_value())
    hi = GRID[GRID >= T]
    lo = GRID[GRID <= -T]
    assert np.all(phi_hat(hi) == 1.0) and np.all(phi_hat(lo) == 0.0)
    assert np.all(gelu_hat(hi) == hi) and np.all(gelu_hat(lo) == 0.0)


def test_center_values():
    z0 = np.zeros(1, np.float32)
    assert phi_hat(z0)[0] == 0.5 and gelu_grad_hat(z0)[0] == 0.5 and gelu_hat(z0)[0] == 0.0
    # leading coefficients are the Taylor ones: φ(0) and 2φ(0)
    assert abs(float(coefficients("kPhiPoly")[0]) - 1 / np.sqrt(2 * np.pi)) < 1e-3
    assert abs(float(coefficients("kGeluGradPoly")[0]) - 2 / np.sqrt(2 * np.pi)) < 1e-3


def test_gelu_grad_error_bound():
    z = GRID.astype(np.float64)
    assert np.abs(gelu_grad_hat(GRID) - gelu_grad(z)).max() <= 1.5e-4


def test_symmetry():
    z = np.linspace(0.0, 6.0, 10001, dtype=np.float32)
    # Φ̂(z) + Φ̂(−z) = 1 up to fp32 rounding of the final fma
    assert np.abs(phi_hat(z) + phi_hat(-z) - 1.0).max() <= 1.2e-7
