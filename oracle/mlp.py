"""fp64 oracle of the Megatron tensor-parallel MLP shard (test infrastructure).

The layer is O = φ(X·A)·B with X [n, d], A [d, m], B [m, d] and φ the exact
erf GeLU.  Tensor parallelism splits A into t column blocks A_i and B into the
matching t row blocks B_i, so that

    O = Σ_i φ(X·A_i)·B_i                      ([TUT] §二, first display;
                                               [SENSE] §2.1 Eq.(1) and Eq.(2))

Shard i computes Z_i = X·A_i, Y_i = φ(Z_i), P_i = Y_i·B_i, and for the upstream
gradient G = ∂ℓ/∂O

    D_i   = (G·B_iᵀ) ⊙ φ'(Z_i)
    dA_i  = Xᵀ·D_i,   dB_i = Y_iᵀ·G,   dX = Σ_i D_i·A_iᵀ
                                              ([TUT] §二 "前向少通信，反向为何仍要
                                               一次归约？")

The sum over shards of P_i (forward) and of dX_i = D_i·A_iᵀ (backward) is what
an all-reduce computes across GPUs ([TRAIN] RowParallelLinear / Column-
ParallelLinear sections: forward all_reduce after the row-parallel matmul,
backward all_reduce of the column-parallel input gradient).  Here it is a
plain fp64 sum; the pages allow any summation order ([TUT] §二: order may
differ, no gradient term may be lost) and ask for a sum, never a mean, over
the group ([TUT] §三).
"""

import numpy as np
from scipy.special import erf

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


# ---------------------------------------------------------------- activation
def gelu(z):
    """Exact GeLU φ(z) = z·Φ(z) = ½·z·(1 + erf(z/√2)).

    The pages name GeLU without printing it ([TRAIN] 激活函数 section: torch
    gelu or TE; [EFF] §4.2 fused bias+GeLU).  The exact (erf) form is the one
    torch.nn.functional.gelu computes by default; the tanh approximation is
    not used anywhere.
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + erf(z / _SQRT2))


def gelu_prime(z):
    """dφ/dz = Φ(z) + z·ϕ(z), with ϕ the standard normal density.

    [TRAIN] 激活函数 section: the activation is a scalar function and is
    differentiated as one.
    """
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / _SQRT2)) + z * np.exp(-0.5 * z * z) * _INV_SQRT_2PI


def relu(z):
    """ReLU, used only by the counterexample of [TUT] §二 教学算例."""
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def relu_prime(z):
    return (np.asarray(z, dtype=np.float64) > 0.0).astype(np.float64)


ACTIVATIONS = {"gelu": (gelu, gelu_prime), "relu": (relu, relu_prime)}


# ---------------------------------------------------------------- sharding
def split_columns(A, t):
    """A [d, m] -> t contiguous column blocks A_i [d, m/t].

    [SENSE] §2.1: splits are even ("切分都是指均分"); [TUT] §二 给两次投影标上跨卡
    尺寸: a 4×8 first weight becomes two 4×4 column blocks.
    """
    A = np.asarray(A, dtype=np.float64)
    m = A.shape[1]
    if t < 1 or m % t:
        raise ValueError(f"hidden width {m} is not divisible by t={t}")
    mi = m // t
    return [A[:, i * mi:(i + 1) * mi] for i in range(t)]


def split_rows(B, t):
    """B [m, d] -> t contiguous row blocks B_i [m/t, d] (same source as
    split_columns: an 8×4 second weight becomes two 4×4 row blocks)."""
    B = np.asarray(B, dtype=np.float64)
    m = B.shape[0]
    if t < 1 or m % t:
        raise ValueError(f"hidden width {m} is not divisible by t={t}")
    mi = m // t
    return [B[i * mi:(i + 1) * mi, :] for i in range(t)]


# ---------------------------------------------------------------- one shard
def shard_forward(X, A_i, B_i, act="gelu"):
    """Z_i = X·A_i, Y_i = φ(Z_i), P_i = Y_i·B_i  ([TUT] §二)."""
    f, _ = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    Z = X @ np.asarray(A_i, dtype=np.float64)
    Y = f(Z)
    P = Y @ np.asarray(B_i, dtype=np.float64)
    return Z, Y, P


def shard_backward(X, A_i, B_i, Z, Y, G, act="gelu"):
    """D_i = (G·B_iᵀ)⊙φ'(Z_i), dA_i = Xᵀ·D_i, dB_i = Y_iᵀ·G, dX_i = D_i·A_iᵀ.

    [TUT] §二 "前向少通信，反向为何仍要一次归约？" gives the first three; the
    input-gradient contribution D_i·A_iᵀ is the summand of ∂ℓ/∂X there.
    Returns (D, dA, dB, dX_i).
    """
    _, fp = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    A_i = np.asarray(A_i, dtype=np.float64)
    B_i = np.asarray(B_i, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    E = G @ B_i.T
    D = E * fp(np.asarray(Z, dtype=np.float64))
    dA = X.T @ D
    dB = np.asarray(Y, dtype=np.float64).T @ G
    dXi = D @ A_i.T
    return D, dA, dB, dXi


def reduce_partials(partials):
    """Σ_i partial_i (the one-GPU stand-in for the all-reduce; a sum, not a
    mean, [TUT] §三)."""
    out = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        out = out + np.asarray(p, dtype=np.float64)
    return out


# ---------------------------------------------------------------- all shards
def tp_forward(X, A, B, t, act="gelu"):
    """Forward of all t shards from the full weights, plus O = Σ_i P_i."""
    A_s, B_s = split_columns(A, t), split_rows(B, t)
    Z, Y, P = [], [], []
    for i in range(t):
        z, y, p = shard_forward(X, A_s[i], B_s[i], act)
        Z.append(z), Y.append(y), P.append(p)
    return {"Z": Z, "Y": Y, "P": P, "O": reduce_partials(P)}


def tp_backward(X, A, B, fwd, G, act="gelu"):
    """Backward of all t shards; dX = Σ_i dX_i."""
    t = len(fwd["Z"])
    A_s, B_s = split_columns(A, t), split_rows(B, t)
    D, dA, dB, dXp = [], [], [], []
    for i in range(t):
        d_, da, db, dx = shard_backward(X, A_s[i], B_s[i], fwd["Z"][i], fwd["Y"][i], G, act)
        D.append(d_), dA.append(da), dB.append(db), dXp.append(dx)
    return {"D": D, "dA": dA, "dB": dB, "dXp": dXp, "dX": reduce_partials(dXp)}


# ---------------------------------------------------------------- unsharded
def dense_forward(X, A, B, act="gelu"):
    """The unsharded layer O = φ(X·A)·B ([TUT] §二, Y = f(XA)B)."""
    f, _ = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    return f(X @ np.asarray(A, dtype=np.float64)) @ np.asarray(B, dtype=np.float64)


def dense_backward(X, A, B, G, act="gelu"):
    """Gradients of ℓ = Σ G⊙O for the unsharded layer by the chain rule:
    H = X·A, ∂ℓ/∂H = (G·Bᵀ)⊙φ'(H), then the matmul rules grad_left = g·rightᵀ
    and grad_right = leftᵀ·g ([TRAIN] custom autograd.Function C = A@B).
    Returns (dX, dA, dB)."""
    f, fp = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    H = X @ A
    dH = (G @ B.T) * fp(H)
    return dH @ A.T, X.T @ dH, f(H).T @ G


# ---------------------------------------------------------------- the wrong split
def row_first_split_forward(X, A, B, t, act="gelu"):
    """The split the pages warn against ([TUT] §二 教学算例 and the paragraph
    after it): cut the *input* channels (rows of A, columns of X), apply the
    activation to each partial sum, then add.  It is NOT the method; tests use
    it to show that φ(u+v) ≠ φ(u)+φ(v) makes it wrong."""
    f, _ = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    d = A.shape[0]
    if d % t:
        raise ValueError("input width not divisible by t")
    di = d // t
    acc = np.zeros((X.shape[0], A.shape[1]))
    for i in range(t):
        acc = acc + f(X[:, i * di:(i + 1) * di] @ A[i * di:(i + 1) * di, :])
    return acc @ np.asarray(B, dtype=np.float64)


def loss(O, G):
    """ℓ = Σ G⊙O, the scalar whose gradient with respect to O is G."""
    return float(np.sum(np.asarray(G, dtype=np.float64) * np.asarray(O, dtype=np.float64)))
