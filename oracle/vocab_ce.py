"""fp64 oracle of the vocabulary-parallel cross-entropy head (test
infrastructure: only tests/, the smoke check and the benchmark's CPU baseline
use it; the product path never does).

The logit layer maps hidden states X [n, h] to the vocabulary with the
embedding table W [V, h]: logits = X·Wᵀ [n, V]; its FLOPs are 2·n·h·V forward
and twice that backward ([EFF] FLOPs appendix, the logit-layer item).  Tensor
parallelism splits the vocabulary: shard i owns rows [i·V/t, (i+1)·V/t) of W
and computes its own logit columns, and the cross-entropy is formed without
gathering them ([SENSE] §2.2.2, Eq. (3) and (4)):

    per shard i and token r:  m_i = max_k x_k (over the shard's columns),
                              s_i = Σ_k exp(x_k − m_i),
                              τ_i = x_target if the target column is the
                                    shard's, else 0
    m = max_i m_i             (the first small all-reduce: a max)
    S = Σ_i s_i·exp(m_i − m)  (the second: a sum; Eq. (3) with x_max of Eq. (4))
    τ = Σ_i τ_i               (the third: a sum)
    loss_r = ln S + m − τ

which equals logsumexp(x) − x_target of the unsplit row.  Backward, for an
upstream gradient g_r = ∂ℓ/∂loss_r:

    dlogits[r, k] = g_r·(exp(x_k − m)/S − [k = target_r])
    dX = dlogits·W,   dW = dlogitsᵀ·X

The combine step is written out as the three reductions above, each over the
shards in order.
"""

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def split_vocab(W, t):
    """W [V, h] -> t contiguous row blocks [V/t, h]."""
    W = _f64(W)
    V = W.shape[0]
    if t < 1 or V % t:
        raise ValueError(f"vocabulary {V} is not divisible by t={t}")
    vi = V // t
    return [W[i * vi:(i + 1) * vi] for i in range(t)]


def shard_logits(X, W_i):
    return _f64(X) @ _f64(W_i).T


def shard_stats(logits_i, targets, start):
    """Per token: the shard's max, its sum of exp(x − max) and its target logit
    (0 where the target is another shard's)."""
    L = _f64(logits_i)
    n, vi = L.shape
    m = L.max(axis=1)
    s = np.exp(L - m[:, None]).sum(axis=1)
    tau = np.zeros(n)
    for r in range(n):
        k = int(targets[r]) - start
        if 0 <= k < vi:
            tau[r] = L[r, k]
    return m, s, tau


def combine(stats):
    """The three reductions over the shards' (m_i, s_i, τ_i)."""
    m = stats[0][0].copy()
    for mi, _, _ in stats[1:]:
        m = np.maximum(m, mi)
    S = np.zeros_like(m)
    tau = np.zeros_like(m)
    for mi, si, ti in stats:
        S = S + si * np.exp(mi - m)
        tau = tau + ti
    return m, S, np.log(S) + m - tau


def tp_forward(X, W, targets, t):
    """logits of every shard, the per-shard statistics and the combined loss."""
    W_s = split_vocab(W, t)
    vi = W_s[0].shape[0]
    logits = [shard_logits(X, W_s[i]) for i in range(t)]
    stats = [shard_stats(logits[i], targets, i * vi) for i in range(t)]
    m, S, loss = combine(stats)
    return {"logits": logits, "stats": stats, "max": m, "sum": S, "loss": loss, "t": t}


def tp_backward(X, W, targets, fwd, g):
    """dlogits of every shard, dX (the sum over shards of dlogits_i·W_i) and
    each shard's dW_i = dlogits_iᵀ·X."""
    X, g = _f64(X), _f64(g)
    t = fwd["t"]
    W_s = split_vocab(W, t)
    vi = W_s[0].shape[0]
    dlog, dW = [], []
    dX = np.zeros_like(X)
    for i in range(t):
        P = np.exp(fwd["logits"][i] - fwd["max"][:, None]) / fwd["sum"][:, None]
        for r in range(X.shape[0]):
            k = int(targets[r]) - i * vi
            if 0 <= k < vi:
                P[r, k] -= 1.0
        D = P * g[:, None]
        dlog.append(D)
        dX = dX + D @ W_s[i]
        dW.append(D.T @ X)
    return {"dlogits": dlog, "dX": dX, "dW": dW}


def dense_loss(X, W, targets):
    """The unsplit definition: logsumexp of each logit row minus its target."""
    L = _f64(X) @ _f64(W).T
    mx = L.max(axis=1, keepdims=True)
    lse = (mx + np.log(np.exp(L - mx).sum(axis=1, keepdims=True)))[:, 0]
    return lse - L[np.arange(L.shape[0]), np.asarray(targets, dtype=np.int64)]
