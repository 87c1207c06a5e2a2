"""fp64 oracle of the Megatron tensor-parallel self-attention shard (test
infrastructure: only tests/, the smoke check and the benchmark's CPU baseline
use it; the product path never does).

The layer: X [n, d] holds n = s·b tokens in [s, b] order (row s_idx·b + b_idx,
the sequence-first layout of [EFF] §4.2), a heads of width dh = d / a.

    QKV = X·W_qkv            W_qkv [d, 3d], columns ordered (head, q|k|v, dh)
    per head h and batch entry β, with q, k, v [s, dh] its slices:
        S = q·kᵀ / √dh       ([TRAIN] Attention 层 section)
        S[i][j] = −∞ for j > i when the mask is causal (GPT; [EFF] §4.2: the
                                 implicit causal mask of the fused softmax)
        S[i][j] = −∞ where a general mask hides key j from query i (the
                                 fused softmax's other kernel in [EFF] §4.2,
                                 for masks like BERT's; [TRAIN]'s BERT layer
                                 uses the padding mask type); mask[β] is one
                                 [s, s] boolean array shared by all heads and
                                 shards, combined with the causal one
        a row whose keys are all hidden has o = 0, no softmax (A = 0) and
                                 lse = −∞, so it passes no gradient
        A = softmax(S) over each row ([TRAIN] Attention 层 section)
        o = A·v
    Ocat = the heads' o side by side, [n, d] in (head, dh) column order
    Out = Ocat·W_proj        W_proj [d, d]

Tensor parallelism splits the heads: shard i of t owns a/t consecutive heads,
i.e. the contiguous column block i of W_qkv (column-parallel, no gather) and
the matching row block i of W_proj (row-parallel, input already split); the
heads interact only inside the shard, so Out = Σ_i Ocat_i·W_proj,i and the sum
is the layer's one forward all-reduce ([SENSE] §2.1.1, the multi-head
attention paragraph and its module: qkv column-parallel with
gather_output=False, proj row-parallel with input_is_parallel=True, per-shard
head count a/t).  The per-head column order (q, k, v adjacent for each head)
follows that module's reshape of the qkv output to (heads, 3, dh).

Backward, for the upstream gradient G = ∂ℓ/∂Out:
    dOcat_i = G·W_proj,iᵀ,   dW_proj,i = Ocat_iᵀ·G
    per head: dv = Aᵀ·do,  dA = do·vᵀ,
              dS = A ⊙ (dA − rowsum(dA ⊙ A))      (softmax gradient, [TRAIN]
                                                   Attention 层 section)
              dq = dS·k/√dh,  dk = dSᵀ·q/√dh
    dQKV_i assembled like QKV_i,  dW_qkv,i = Xᵀ·dQKV_i,  dX_i = dQKV_i·W_qkv,iᵀ
and dX = Σ_i dX_i (the backward all-reduce of the column-parallel input).

Optional biases as for the MLP ([TRAIN] ColumnParallelLinear / RowParallel-
Linear): b_qkv split like W_qkv's columns and added to QKV_i; b_proj unsplit,
added once after the sum.  The attention dropout is not applied: the module on
[SENSE] defaults it to 0.

Everything is plain NumPy in fp64 with a loop over (batch entry, head); the
softmax subtracts the row maximum first (any constant cancels).  lse is the
natural log of each row's Σ exp(S), the statistic the GPU path keeps for its
backward.
"""

import numpy as np

from . import mlp as _mlp


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- head layout
def split_heads(QKV, s, b, nh, dh):
    """QKV [s·b, nh·3·dh] -> q, k, v, each [b, nh, s, dh]."""
    T = _f64(QKV).reshape(s, b, nh, 3, dh)
    q = T[:, :, :, 0, :].transpose(1, 2, 0, 3)
    k = T[:, :, :, 1, :].transpose(1, 2, 0, 3)
    v = T[:, :, :, 2, :].transpose(1, 2, 0, 3)
    return q, k, v


def merge_qkv(dq, dk, dv):
    """Inverse of split_heads: three [b, nh, s, dh] -> [s·b, nh·3·dh]."""
    b, nh, s, dh = dq.shape
    T = np.stack([dq, dk, dv], axis=3)          # [b, nh, s, 3, dh]
    return T.transpose(2, 0, 1, 3, 4).reshape(s * b, nh * 3 * dh)


def merge_heads(o):
    """[b, nh, s, dh] -> Ocat [s·b, nh·dh] in (head, dh) column order."""
    b, nh, s, dh = o.shape
    return o.transpose(2, 0, 1, 3).reshape(s * b, nh * dh)


def unmerge_heads(Ocat, s, b, nh, dh):
    return _f64(Ocat).reshape(s, b, nh, dh).transpose(1, 2, 0, 3)


# ---------------------------------------------------------------- the core
def core_forward(q, k, v, causal, mask=None):
    """Per (batch entry, head): S = q·kᵀ/√dh, causal and/or general mask
    (mask [b, s, s], True hides key j from query i), row softmax, o = A·v.
    Returns o [b, nh, s, dh], A [b, nh, s, s], lse [b, nh, s]; rows with every
    key hidden get o = 0, A = 0, lse = −∞."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, nh, s, dh = q.shape
    scale = 1.0 / np.sqrt(dh)
    o = np.zeros_like(q)
    A = np.zeros((b, nh, s, s))
    lse = np.zeros((b, nh, s))
    base = np.tril(np.ones((s, s), dtype=bool)) if causal else np.ones((s, s), dtype=bool)
    for bi in range(b):
        keep = base if mask is None else base & ~np.asarray(mask[bi], dtype=bool)
        seen = keep.any(axis=1)
        for h in range(nh):
            S = (q[bi, h] @ k[bi, h].T) * scale
            S = np.where(keep, S, -np.inf)
            mx = np.where(seen, S.max(axis=1), 0.0)[:, None]
            E = np.exp(S - mx)
            z = E.sum(axis=1, keepdims=True)
            A[bi, h] = np.where(seen[:, None], E / np.where(seen[:, None], z, 1.0), 0.0)
            lse[bi, h] = np.where(seen, mx[:, 0] + np.log(np.where(seen, z[:, 0], 1.0)), -np.inf)
            o[bi, h] = A[bi, h] @ v[bi, h]
    return o, A, lse


def core_backward(q, k, v, A, do):
    """Gradients of the core for the upstream do [b, nh, s, dh]."""
    q, k, v, A, do = _f64(q), _f64(k), _f64(v), _f64(A), _f64(do)
    b, nh, s, dh = q.shape
    scale = 1.0 / np.sqrt(dh)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for bi in range(b):
        for h in range(nh):
            P = A[bi, h]
            dv[bi, h] = P.T @ do[bi, h]
            dP = do[bi, h] @ v[bi, h].T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            dq[bi, h] = (dS @ k[bi, h]) * scale
            dk[bi, h] = (dS.T @ q[bi, h]) * scale
    return dq, dk, dv


# ---------------------------------------------------------------- one shard
def shard_forward(X, Wqkv_i, Wproj_i, s, b, nh, causal, bqkv_i=None, mask=None):
    """QKV_i = X·W_qkv,i (+ bqkv_i), the core on the shard's nh heads,
    P_i = Ocat_i·W_proj,i."""
    X = _f64(X)
    dh = Wqkv_i.shape[1] // (3 * nh)
    QKV = X @ _f64(Wqkv_i)
    if bqkv_i is not None:
        QKV = QKV + _f64(bqkv_i)[None, :]
    q, k, v = split_heads(QKV, s, b, nh, dh)
    o, A, lse = core_forward(q, k, v, causal, mask)
    Ocat = merge_heads(o)
    P = Ocat @ _f64(Wproj_i)
    return {"QKV": QKV, "A": A, "lse": lse, "O": Ocat, "P": P}


def shard_backward(X, Wqkv_i, Wproj_i, fwd, G, s, b, nh):
    """dOcat_i, dW_proj,i, the core's gradients, dQKV_i, dW_qkv,i, dX_i (and
    the shard's q/k/v bias gradient, Σ_rows dQKV_i)."""
    X, G = _f64(X), _f64(G)
    Wqkv_i, Wproj_i = _f64(Wqkv_i), _f64(Wproj_i)
    dh = Wqkv_i.shape[1] // (3 * nh)
    dO = G @ Wproj_i.T
    dWproj = fwd["O"].T @ G
    q, k, v = split_heads(fwd["QKV"], s, b, nh, dh)
    dq, dk, dv = core_backward(q, k, v, fwd["A"], unmerge_heads(dO, s, b, nh, dh))
    dQKV = merge_qkv(dq, dk, dv)
    dWqkv = X.T @ dQKV
    dXi = dQKV @ Wqkv_i.T
    return {"dO": dO, "dWproj": dWproj, "dQKV": dQKV, "dWqkv": dWqkv, "dXp": dXi,
            "dbqkv": _mlp.bias_grad(dQKV)}


# ---------------------------------------------------------------- all shards
def tp_forward(X, Wqkv, Wproj, t, s, b, heads, causal, bqkv=None, bproj=None, mask=None):
    """All t shards from the full weights (heads/t heads each) and
    Out = Σ_i P_i (+ bproj once after the sum)."""
    if heads % t:
        raise ValueError(f"{heads} heads are not divisible by t={t}")
    nh = heads // t
    Wq_s = _mlp.split_columns(Wqkv, t)
    Wp_s = _mlp.split_rows(Wproj, t)
    bq_s = _mlp.split_bias(bqkv, t) if bqkv is not None else [None] * t
    shards = [shard_forward(X, Wq_s[i], Wp_s[i], s, b, nh, causal, bq_s[i], mask) for i in range(t)]
    Out = _mlp.reduce_partials([sh["P"] for sh in shards])
    if bproj is not None:
        Out = Out + _f64(bproj)[None, :]
    return {"shards": shards, "Out": Out, "t": t, "nh": nh, "s": s, "b": b}


def tp_backward(X, Wqkv, Wproj, fwd, G):
    t, nh, s, b = fwd["t"], fwd["nh"], fwd["s"], fwd["b"]
    Wq_s = _mlp.split_columns(Wqkv, t)
    Wp_s = _mlp.split_rows(Wproj, t)
    shards = [shard_backward(X, Wq_s[i], Wp_s[i], fwd["shards"][i], G, s, b, nh) for i in range(t)]
    return {"shards": shards, "dX": _mlp.reduce_partials([sh["dXp"] for sh in shards]),
            "dbproj": _mlp.bias_grad(G)}
