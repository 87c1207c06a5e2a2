"""fp64 oracle of LayerNorm forward and backward (test infrastructure).

[TRAIN] LayerNorm section: per token x ∈ R^h, take the mean and variance,
centre and normalise, then apply the learned scale γ and shift β.  Backward:
with g = ∂L/∂y and g̃ = g⊙γ, the input gradient is g̃ with its components along
the all-ones direction and along x̂ removed, scaled by 1/σ; the page notes that
the result is orthogonal to both 𝟏 and x̂.

The page's display formulas are missing from the text; the reading taken is
that of torch.nn.LayerNorm, which the page names: biased variance over h and
eps inside the square root.
"""

import numpy as np


def ln_forward(x, gamma, beta, eps):
    """Row-wise LayerNorm of x [rows, h].  Returns (y, mean, rstd, xhat)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean[:, None]) * rstd[:, None]
    y = xhat * np.asarray(gamma, dtype=np.float64)[None, :] + np.asarray(beta, dtype=np.float64)[None, :]
    return y, mean, rstd, xhat


def ln_backward(g, xhat, rstd, gamma):
    """Gradients of a row-wise LayerNorm.

    g̃ = g⊙γ;  dx = rstd·(g̃ − mean_j(g̃) − x̂·mean_j(g̃⊙x̂));
    dγ = Σ_rows g⊙x̂;  dβ = Σ_rows g.      Returns (dx, dgamma, dbeta).
    """
    g = np.asarray(g, dtype=np.float64)
    gt = g * np.asarray(gamma, dtype=np.float64)[None, :]
    proj1 = gt.mean(axis=1, keepdims=True)
    projx = (gt * xhat).mean(axis=1, keepdims=True)
    dx = rstd[:, None] * (gt - proj1 - xhat * projx)
    return dx, (g * xhat).sum(axis=0), g.sum(axis=0)
