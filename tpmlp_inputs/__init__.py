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
  * The attention side (attn_inputs): X [s·b, d], W_qkv [d, 3d], W_proj
    [d, d], G [s·b, d] drawn in that order with the same deviations; its
    optional biases from default_rng([seed, 2]).
  * The logit layer (vocab_inputs): X [n, h], W [V, h], targets uniform in
    [0, V), g [n] (the upstream gradient of each token's loss; the mean loss
    over n tokens has g = 1/n), drawn in that order.
  * Biases b1 [m], b2 [d] (bias_inputs) come from a stream of their own,
    default_rng([seed, 1]), with std 0.5.
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
    # attention side of the GPT-8.3B-shaped layer: h=3072, 24 heads of 128,
    # t=8 (3 heads per shard), b=8, s=1024 tokens per sequence, causal.
    "gpt8p3b_attn_t8": dict(kind="attn", s=1024, b=8, d=3072, heads=24, t=8, dtype="bf16",
                            causal=True, x_std=X_STD, w_std=W_STD, g_std=G_STD),
    # logit layer + cross-entropy of the 8.3B-shaped model: h=3072, a padded
    # GPT-2 vocabulary V=51200 (50257 rounded up to a multiple of 1024), t=8
    # (6400 entries per shard), n=b·s=8·1024 tokens.
    "gpt8p3b_vocab_t8": dict(kind="vocab", n=8192, d=3072, V=51200, t=8, dtype="bf16",
                             x_std=X_STD, w_std=W_STD, g_std=1.0 / 8192),
    # sequence-parallel block: s=4096, h=4096, m=4h, t=8, LN + dropout 0.1.
    "sp_block_t8": dict(kind="sp", n=4096, d=4096, m=16384, t=8, dtype="bf16",
                        x_std=X_STD, w_std=W_STD, g_std=G_STD,
                        gamma_std=0.1, beta_std=0.1, eps=1e-5, p=0.1, mask_seed=0),
}


def f32_to_bf16_bits(x):
    """Round finite fp32 values to bf16 (nearest-even); returns uint16 bit
    patterns.  (No finite input can overflow the 32-bit sum.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK = 1 << 22  # elements drawn per step (the stream does not depend on it)


def _draw(rng, shape, std, dtype):
    """standard_normal fp64 × std, rounded to the storage dtype chunk by chunk;
    returns fp32 values or bf16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(0, n, _CHUNK):
        v32 = (rng.standard_normal(min(_CHUNK, n - b)) * std).astype(np.float32)
        out[b:b + v32.size] = f32_to_bf16_bits(v32) if dtype == "bf16" else v32
    return out.reshape(shape)


class Tensor:
    """One synthetic tensor: the stored values (fp32, or bf16 bit patterns)
    and, on demand, the same values upcast exactly to fp32 / fp64."""

    def __init__(self, stored, dtype):
        if dtype not in ("bf16", "f32"):
            raise ValueError(dtype)
        self.dtype = dtype
        self.bits = stored if dtype == "bf16" else None
        self._f32 = None if dtype == "bf16" else stored
        self.shape = stored.shape

    @property
    def f32(self):
        if self._f32 is None:
            self._f32 = bf16_bits_to_f32(self.bits)
        return self._f32

    @property
    def f64(self):
        return self.f32.astype(np.float64)


def mlp_inputs(n, d, m, t, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD,
               g_std=G_STD, shards=None):
    """X [n, d], A [d, m] (or shard-0 [d, m/t]), B [m, d] (or [m/t, d]), G [n, d]."""
    if m % t:
        raise ValueError("m must be divisible by t")
    rng = np.random.default_rng(seed)
    mw = m if shards is None else m // t
    X = _draw(rng, (n, d), x_std, dtype)
    A = _draw(rng, (d, mw), w_std, dtype)
    B = _draw(rng, (mw, d), w_std, dtype)
    G = _draw(rng, (n, d), g_std, dtype)
    return {"X": Tensor(X, dtype), "A": Tensor(A, dtype), "B": Tensor(B, dtype),
            "G": Tensor(G, dtype)}


def sp_inputs(s, h, m, t, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD,
              g_std=G_STD, gamma_std=0.1, beta_std=0.1):
    """x [s, h], A [h, m], B [m, h], G_out [s, h], γ = 1 + N(0, σ²), β = N(0, σ²)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (s, h), x_std, dtype)
    A = _draw(rng, (h, m), w_std, dtype)
    B = _draw(rng, (m, h), w_std, dtype)
    G = _draw(rng, (s, h), g_std, dtype)
    g32 = (1.0 + rng.standard_normal(h) * gamma_std).astype(np.float32)
    b32 = (rng.standard_normal(h) * beta_std).astype(np.float32)
    gamma = f32_to_bf16_bits(g32) if dtype == "bf16" else g32
    beta = f32_to_bf16_bits(b32) if dtype == "bf16" else b32
    return {"x": Tensor(x, dtype), "A": Tensor(A, dtype), "B": Tensor(B, dtype),
            "G": Tensor(G, dtype), "gamma": Tensor(gamma, dtype), "beta": Tensor(beta, dtype)}


# Bias standard deviation: comparable to the pre-activation spread at the
# workloads' widths (0.02·√3072 ≈ 1.1), so the bias moves GeLU's operating
# point visibly.  (The layers initialise their biases to zero; a zero bias
# would test nothing.)
B_STD = 0.5


def bias_inputs(m, d, dtype="bf16", seed=0, std=B_STD):
    """b1 [m] (the column-parallel layer's bias) and b2 [d] (the row-parallel
    layer's), from their own stream numpy.random.default_rng([seed, 1]) so the
    other tensors' draws are unchanged."""
    rng = np.random.default_rng([seed, 1])
    b1 = _draw(rng, (m,), std, dtype)
    b2 = _draw(rng, (d,), std, dtype)
    return {"b1": Tensor(b1, dtype), "b2": Tensor(b2, dtype)}


def attn_inputs(s, b, d, heads, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD, g_std=G_STD,
                bias_std=None):
    """X [s·b, d] (tokens in [s, b] order), W_qkv [d, 3d], W_proj [d, d],
    G [s·b, d]; with bias_std also b_qkv [3d] and b_proj [d] from the stream
    default_rng([seed, 2])."""
    if d % heads:
        raise ValueError("d must be divisible by the head count")
    rng = np.random.default_rng(seed)
    n = s * b
    X = _draw(rng, (n, d), x_std, dtype)
    Wqkv = _draw(rng, (d, 3 * d), w_std, dtype)
    Wproj = _draw(rng, (d, d), w_std, dtype)
    G = _draw(rng, (n, d), g_std, dtype)
    out = {"X": Tensor(X, dtype), "Wqkv": Tensor(Wqkv, dtype), "Wproj": Tensor(Wproj, dtype),
           "G": Tensor(G, dtype)}
    if bias_std is not None:
        rb = np.random.default_rng([seed, 2])
        out["bqkv"] = Tensor(_draw(rb, (3 * d,), bias_std, dtype), dtype)
        out["bproj"] = Tensor(_draw(rb, (d,), bias_std, dtype), dtype)
    return out


def vocab_inputs(n, h, V, dtype="bf16", seed=0, x_std=X_STD, w_std=W_STD, g_std=1.0):
    """The logit layer: X [n, h], the embedding table W [V, h], integer targets
    [n] uniform in [0, V) (int32), and an upstream gradient per token's loss
    g [n], drawn in that order."""
    rng = np.random.default_rng(seed)
    X = _draw(rng, (n, h), x_std, dtype)
    W = _draw(rng, (V, h), w_std, dtype)
    targets = rng.integers(0, V, size=n).astype(np.int32)
    g = _draw(rng, (n,), g_std, "f32")
    return {"X": Tensor(X, dtype), "W": Tensor(W, dtype), "targets": targets, "g": Tensor(g, "f32")}


def qkv_inputs(T, s, b, nh, dh, dtype="bf16", seed=0, std=1.0):
    """The attention core's inputs alone: qkv [T, s·b, nh·3·dh] and an upstream
    gradient do [T, s·b, nh·dh], both N(0, std²)."""
    rng = np.random.default_rng(seed)
    qkv = _draw(rng, (T, s * b, nh * 3 * dh), std, dtype)
    do = _draw(rng, (T, s * b, nh * dh), std, dtype)
    return {"qkv": Tensor(qkv, dtype), "do": Tensor(do, dtype)}


def attn_mask(b, s, kind="padding", seed=0, p=0.3):
    """A general attention mask [b, s, s] as uint8 (1 hides key j from query
    i), shared by all heads and shards.
      "padding": BERT-style: entry β has a valid length L_β drawn uniformly
                 from [⌈s/2⌉, s]; a position is hidden when the query or the
                 key is at or past L_β (padded query rows see no key)
      "random":  each entry hidden with probability p (rows may end up with
                 no visible key)"""
    rng = np.random.default_rng([seed, 3])
    if kind == "padding":
        L = rng.integers((s + 1) // 2, s + 1, size=b)
        pos = np.arange(s)
        m = (pos[None, :, None] >= L[:, None, None]) | (pos[None, None, :] >= L[:, None, None])
    elif kind == "random":
        m = rng.random((b, s, s)) < p
    else:
        raise ValueError(kind)
    return m.astype(np.uint8)


def config_inputs(name, seed=0):
    c = CONFIGS[name]
    if c["kind"] == "vocab":
        return vocab_inputs(c["n"], c["d"], c["V"], c["dtype"], seed, c["x_std"], c["w_std"], c["g_std"])
    if c["kind"] == "attn":
        return attn_inputs(c["s"], c["b"], c["d"], c["heads"], c["dtype"], seed, c["x_std"],
                           c["w_std"], c["g_std"])
    if c["kind"] == "mlp":
        return mlp_inputs(c["n"], c["d"], c["m"], c["t"], c["dtype"], seed, c["x_std"],
                          c["w_std"], c["g_std"], c.get("shards"))
    return sp_inputs(c["n"], c["d"], c["m"], c["t"], c["dtype"], seed, c["x_std"],
                     c["w_std"], c["g_std"], c["gamma_std"], c["beta_std"])
