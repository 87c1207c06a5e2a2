"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the MLP / LayerNorm / dropout arithmetic, so that neither the oracle
nor the HIP path depends on the other through it.

Recipe (the workloads of the tensor-parallel MLP shard, no dataset involved):
  * numpy.random.default_rng(seed) (PCG64), standard_normal in fp64, scaled by
    the stated standard deviation, drawn in the order X, A (full [d, m]),
    B (full [m, d]), G, then for the sequence-parallel block γ and β.
  * The trillion-parameter-shaped case draws shard 0's A_0 [d, m/t] and
    B_0 [m/t, d] directly (the full A would not fit in host memory).
  * fp64 -> fp32 by round-to-nearest-even (numpy), fp32 -> bf16 by
    round-to-nearest-even on the bit pattern.  The oracle receives the rounded
    values upcast exactly to fp64.
"""

import numpy as np

# Standard deviations; "N(0, 1e-4)" for G is read as variance 1e-4 (std 0.01),
# matching how the weights are written as N(0, 0.02²).
X_STD, W_STD, G_STD = 1.0, 0.02, 0.01

CONFIGS = {
    # fp32 worked example: X 3×4, A 4×8, B 8×4, two shards of 4×4 blocks.
    "worked_example": dict(kind="mlp", n=3, d=4, m=8, t=2, dtype="f32",
                           x_std=1.0, w_std=1.0, g_std=1.0),
    # single-shard bf16 MLP: tokens 4·512, d=1024, m=4096.
    "single_shard": dict(kind="mlp", n=2048, d=1024, m=4096, t=1, dtype="bf16",
                         x_std=X_STD, w_std=W_STD, g_std=G_STD),
    # GPT-8.3B-shaped layer: h=3072, m=4h, t=8, b·s = 8·1024 tokens.
    "gpt8p3b_t8": dict(kind="mlp", n=8192, d=3072, m=12288, t=8, dtype="bf16",
                       x_std=X_STD, w_std=W_STD, g_std=G_STD),
    # trillion-parameter-shaped layer: h=25600, m=4h, t=8, 2048 tokens, shard 0.
    "gpt1t_t8_shard0": dict(kind="mlp", n=2048, d=25600, m=102400, t=8, dtype="bf16",
                            x_std=X_STD, w_std=W_STD, g_std=G_STD, shards=(0,)),
    # sequence-parallel block: s=4096, h=4096, m=4h, t=8, LN + dropout 0.1.
    "sp_block_t8": dict(kind="sp", n=4096, d=4096, m=16384, t=8, dtype="bf16",
                        x_std=X_STD, w_std=W_STD, g_std=G_STD,
                        gamma_std=0.1, beta_std=0.1, eps=1e-5, p=0.1, mask_seed=0),
}


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """One synthetic tensor: the stored values (fp32 or bf16 bits) and the
    same values upcast exactly to fp64 for the oracle."""

    def __init__(self, values64, dtype):
        v32 = np.asarray(values64, dtype=np.float64).astype(np.float32)
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = f32_to_bf16_bits(v32)
            self.f32 = bf16_bits_to_f32(self.bits)
        elif dtype == "f32":
            self.bits = None
            self.f32 = v32
        else:
            raise ValueError(dtype)
        self.shape = self.f32.shape

    @property
    def f64(self):
        return self.f32.astype(np.float64)


def mlp_inputs(n, d, m, t, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD,
               g_std=G_STD, shards=None):
    """X [n, d], A [d, m] (or shard-0 [d, m/t]), B [m, d] (or [m/t, d]), G [n, d]."""
    if m % t:
        raise ValueError("m must be divisible by t")
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, d)) * x_std
    if shards is None:
        A = rng.standard_normal((d, m)) * w_std
        B = rng.standard_normal((m, d)) * w_std
    else:
        mi = m // t
        A = rng.standard_normal((d, mi)) * w_std
        B = rng.standard_normal((mi, d)) * w_std
    G = rng.standard_normal((n, d)) * g_std
    return {"X": Tensor(X, dtype), "A": Tensor(A, dtype), "B": Tensor(B, dtype),
            "G": Tensor(G, dtype)}


def sp_inputs(s, h, m, t, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD,
              g_std=G_STD, gamma_std=0.1, beta_std=0.1):
    """x [s, h], A [h, m], B [m, h], G_out [s, h], γ = 1 + N(0, σ²), β = N(0, σ²)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((s, h)) * x_std
    A = rng.standard_normal((h, m)) * w_std
    B = rng.standard_normal((m, h)) * w_std
    G = rng.standard_normal((s, h)) * g_std
    gamma = 1.0 + rng.standard_normal(h) * gamma_std
    beta = rng.standard_normal(h) * beta_std
    return {"x": Tensor(x, dtype), "A": Tensor(A, dtype), "B": Tensor(B, dtype),
            "G": Tensor(G, dtype), "gamma": Tensor(gamma, dtype), "beta": Tensor(beta, dtype)}


def config_inputs(name, seed=0):
    c = CONFIGS[name]
    if c["kind"] == "mlp":
        return mlp_inputs(c["n"], c["d"], c["m"], c["t"], c["dtype"], seed, c["x_std"],
                          c["w_std"], c["g_std"], c.get("shards"))
    return sp_inputs(c["n"], c["d"], c["m"], c["t"], c["dtype"], seed, c["x_std"],
                     c["w_std"], c["g_std"], c["gamma_std"], c["beta_std"])
