"""fp64 oracle of one sequence-parallel MLP block (test infrastructure).

[SP] "通信插在层内什么位置？": with sequence parallelism the per-token operators
(LayerNorm, dropout, residual add) run on the rank's s/t rows; g = AllGather
joins the LayerNorm outputs before the column-parallel fc1, and ḡ =
ReduceScatter after the row-parallel fc2 sums the partial outputs and hands each
rank its s/t rows back for dropout + residual.  Backward mirrors it ([EFF]
§3.5.1, "开启 SP 后 backward 流程"): local dropout/residual/LN gradients, an
AllGather of the sliced gradient into the MLP's G, and a ReduceScatter of the
MLP's input gradient.  On one GPU the AllGather is a concatenation and the
ReduceScatter is a sum over shards followed by a row split
(AllReduce ≡ AllGather∘ReduceScatter, [SP] eq. par-spmech-ar-identity).

Block, pre-norm with the residual taken from the LayerNorm input ([TRAIN]
Post-Norm 还是 Pre-Norm section; [SP] placement diagram):
    out = x + dropout_p( Σ_i φ(LN(x)·A_i)·B_i )
With biases (optional): the column-parallel bias b1 inside φ and the
row-parallel bias b2 added after the sum, before dropout — the
bias + dropout + add of [EFF] §4.2:
    out = x + dropout_p( Σ_i φ(LN(x)·A_i + b1_i)·B_i + b2 )
The sequence-parallel degree equals the tensor-parallel degree t and must be
at least 2 ([SP] 工程约束: sequence parallelism requires TP > 1).
"""

import numpy as np

from . import mlp as _mlp
from .layernorm import ln_backward, ln_forward
from .philox import keep_mask


def _check(s, t):
    if t < 2:
        raise ValueError("sequence parallelism requires tensor-parallel degree t >= 2")
    if s % t:
        raise ValueError(f"sequence length {s} is not divisible by t={t}")


def sp_forward(x, gamma, beta, eps, A, B, t, p, seed, b1=None, b2=None):
    """Sharded forward: per-shard LN on s/t rows, concat (AllGather), the t MLP
    shards, sum then split (ReduceScatter; the row bias is added to the sum),
    per-shard dropout + residual."""
    x = np.asarray(x, dtype=np.float64)
    s, h = x.shape
    _check(s, t)
    sl = s // t
    parts = [ln_forward(x[r * sl:(r + 1) * sl], gamma, beta, eps) for r in range(t)]
    U = np.concatenate([q[0] for q in parts], axis=0)
    fwd = _mlp.tp_forward(U, A, B, t, b1=b1, b2=b2)
    scale = 1.0 / (1.0 - p)
    outs, masks = [], []
    for r in range(t):
        S_r = fwd["O"][r * sl:(r + 1) * sl]
        M_r = keep_mask(r * sl, sl, h, p, seed)
        outs.append(x[r * sl:(r + 1) * sl] + M_r * S_r * scale)
        masks.append(M_r)
    return {
        "U": U,
        "mean": np.concatenate([q[1] for q in parts]),
        "rstd": np.concatenate([q[2] for q in parts]),
        "xhat": np.concatenate([q[3] for q in parts], axis=0),
        "mlp": fwd,
        "mask": np.concatenate(masks, axis=0),
        "out": np.concatenate(outs, axis=0),
    }


def sp_backward(fwd, gamma, A, B, G_out, t, p):
    """Sharded backward for ℓ = Σ G_out⊙out.  Returns dict with the MLP's
    G (dS), its backward, dU, dx, dgamma, dbeta."""
    G_out = np.asarray(G_out, dtype=np.float64)
    s, h = G_out.shape
    _check(s, t)
    sl = s // t
    scale = 1.0 / (1.0 - p)
    dS = np.concatenate([G_out[r * sl:(r + 1) * sl] * fwd["mask"][r * sl:(r + 1) * sl] * scale
                         for r in range(t)], axis=0)
    bwd = _mlp.tp_backward(fwd["U"], A, B, fwd["mlp"], dS)  # with biases also db1, db2 = Σ_rows dS
    dxs, dgs, dbs = [], [], []
    for r in range(t):
        rows = slice(r * sl, (r + 1) * sl)
        dx_ln, dg, db = ln_backward(bwd["dX"][rows], fwd["xhat"][rows], fwd["rstd"][rows], gamma)
        dxs.append(G_out[rows] + dx_ln)
        dgs.append(dg), dbs.append(db)
    return {
        "dS": dS,
        "mlp": bwd,
        "dU": bwd["dX"],
        "dx": np.concatenate(dxs, axis=0),
        "dgamma": _mlp.reduce_partials(dgs),
        "dbeta": _mlp.reduce_partials(dbs),
    }


def dense_forward(x, gamma, beta, eps, A, B, p, seed, b1=None, b2=None):
    """The same block with no sharding at all: LN on all rows, the unsharded
    MLP, one mask over the whole [s, h], residual."""
    x = np.asarray(x, dtype=np.float64)
    s, h = x.shape
    U, mean, rstd, xhat = ln_forward(x, gamma, beta, eps)
    S = _mlp.dense_forward(U, A, B, b1=b1, b2=b2)
    M = keep_mask(0, s, h, p, seed)
    return {"U": U, "xhat": xhat, "rstd": rstd, "mask": M, "out": x + M * S / (1.0 - p)}


def dense_backward(fwd, gamma, A, B, G_out, p, b1=None):
    G_out = np.asarray(G_out, dtype=np.float64)
    dS = G_out * fwd["mask"] / (1.0 - p)
    out = {}
    if b1 is None:
        dU, dA, dB = _mlp.dense_backward(fwd["U"], A, B, dS)
    else:
        dU, dA, dB, out["db1"], out["db2"] = _mlp.dense_backward(fwd["U"], A, B, dS, b1=b1)
    dx_ln, dg, db = ln_backward(dU, fwd["xhat"], fwd["rstd"], gamma)
    out.update({"dx": G_out + dx_ln, "dgamma": dg, "dbeta": db, "dA": dA, "dB": dB})
    return out
