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

With the layers' biases ([TRAIN] ColumnParallelLinear: the bias is split like
the output columns, b1_i; RowParallelLinear: one unsplit bias b2 added after
the all-reduce) the shard computes Z_i = X·A_i + b1_i and the layer
O = Σ_i P_i + b2; the bias gradients are the upstream gradients summed over
the tokens ([TRAIN] custom autograd matmul rule, grad_bias = Σ over rows):
db1_i = Σ_rows D_i, db2 = Σ_rows G.

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
def shard_forward(X, A_i, B_i, act="gelu", b1_i=None):
    """Z_i = X·A_i (+ b1_i on every row), Y_i = φ(Z_i), P_i = Y_i·B_i
    ([TUT] §二; the bias per [TRAIN] ColumnParallelLinear)."""
    f, _ = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    Z = X @ np.asarray(A_i, dtype=np.float64)
    if b1_i is not None:
        Z = Z + np.asarray(b1_i, dtype=np.float64)[None, :]
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


def bias_grad(g):
    """Σ over the rows (tokens) of an upstream gradient: the gradient of a bias
    broadcast over those rows ([TRAIN] custom autograd matmul rule)."""
    g = np.asarray(g, dtype=np.float64)
    out = np.zeros(g.shape[1])
    for r in range(g.shape[0]):
        out = out + g[r]
    return out


def split_bias(b1, t):
    """b1 [m] -> t contiguous blocks of m/t, matching the column blocks of A."""
    b1 = np.asarray(b1)
    m = b1.shape[0]
    if m % t:
        raise ValueError(f"bias length {m} is not divisible by t={t}")
    mi = m // t
    return [b1[i * mi:(i + 1) * mi] for i in range(t)]


def reduce_partials(partials):
    """Σ_i partial_i (the one-GPU stand-in for the all-reduce; a sum, not a
    mean, [TUT] §三)."""
    out = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for p in partials:
        out = out + np.asarray(p, dtype=np.float64)
    return out


# ---------------------------------------------------------------- all shards
def tp_forward(X, A, B, t, act="gelu", b1=None, b2=None):
    """Forward of all t shards from the full weights, plus O = Σ_i P_i (+ b2
    on every row, added once after the sum)."""
    A_s, B_s = split_columns(A, t), split_rows(B, t)
    b1_s = split_bias(b1, t) if b1 is not None else [None] * t
    Z, Y, P = [], [], []
    for i in range(t):
        z, y, p = shard_forward(X, A_s[i], B_s[i], act, b1_s[i])
        Z.append(z), Y.append(y), P.append(p)
    O = reduce_partials(P)
    if b2 is not None:
        O = O + np.asarray(b2, dtype=np.float64)[None, :]
    return {"Z": Z, "Y": Y, "P": P, "O": O, "biased": b1 is not None or b2 is not None}


def tp_backward(X, A, B, fwd, G, act="gelu"):
    """Backward of all t shards; dX = Σ_i dX_i."""
    t = len(fwd["Z"])
    A_s, B_s = split_columns(A, t), split_rows(B, t)
    D, dA, dB, dXp = [], [], [], []
    for i in range(t):
        d_, da, db, dx = shard_backward(X, A_s[i], B_s[i], fwd["Z"][i], fwd["Y"][i], G, act)
        D.append(d_), dA.append(da), dB.append(db), dXp.append(dx)
    out = {"D": D, "dA": dA, "dB": dB, "dXp": dXp, "dX": reduce_partials(dXp)}
    if fwd.get("biased"):
        out["db1"] = [bias_grad(d_) for d_ in D]
        out["db2"] = bias_grad(G)
    return out


# ---------------------------------------------------------------- unsharded
def dense_forward(X, A, B, act="gelu", b1=None, b2=None):
    """The unsharded layer O = φ(X·A + b1)·B + b2 ([TUT] §二, Y = f(XA)B; the
    biases broadcast over the rows)."""
    f, _ = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    H = X @ np.asarray(A, dtype=np.float64)
    if b1 is not None:
        H = H + np.asarray(b1, dtype=np.float64)[None, :]
    O = f(H) @ np.asarray(B, dtype=np.float64)
    if b2 is not None:
        O = O + np.asarray(b2, dtype=np.float64)[None, :]
    return O


def dense_backward(X, A, B, G, act="gelu", b1=None):
    """Gradients of ℓ = Σ G⊙O for the unsharded layer by the chain rule:
    H = X·A (+ b1), ∂ℓ/∂H = (G·Bᵀ)⊙φ'(H), then the matmul rules
    grad_left = g·rightᵀ and grad_right = leftᵀ·g ([TRAIN] custom
    autograd.Function C = A@B).  Returns (dX, dA, dB); with b1 given also
    (db1, db2) = (Σ_rows ∂ℓ/∂H, Σ_rows G)."""
    f, fp = ACTIVATIONS[act]
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    H = X @ A
    if b1 is not None:
        H = H + np.asarray(b1, dtype=np.float64)[None, :]
    dH = (G @ B.T) * fp(H)
    if b1 is None:
        return dH @ A.T, X.T @ dH, f(H).T @ G
    return dH @ A.T, X.T @ dH, f(H).T @ G, bias_grad(dH), bias_grad(G)


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
