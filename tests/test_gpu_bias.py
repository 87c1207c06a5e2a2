"""GPU parity of the bias variants through the C ABI against the fp64 oracle
on the same seeded inputs: tpmlp_fwd_bias (bias + GeLU in the first GEMM's
epilogue), tpmlp_reduce_partials_bias (the unsplit second bias after the sum),
tpmlp_bias_grad (db1_i = Σ_rows D_i, db2 = Σ_rows G) and the sequence-parallel
bias + dropout + residual.

Bars (relative Frobenius error, fp64): fp32 path 1e-5, bf16 path 8e-3 for
every output, gradient and stored intermediate; the bias gradient of given
(stored) values is an fp32 column sum, held to 1e-5 on either path.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import mlp as om
from oracle import sp_block as osp
from tpmlp_inputs import CONFIGS, bias_inputs, config_inputs, mlp_inputs, sp_inputs

from gpu_util import dev, f64, relerr, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3}
SUM_TOL = 1e-5


def run_biased_step(X, A_s, B_s, b1_s, b2, G, fused=False):
    """fused: tpmlp_bwd_bias (db1 from the dgrad-1 epilogue, db2 inside the
    call); else tpmlp_bwd and two tpmlp_bias_grad calls."""
    Z, Y, P = tp.mlp_fwd_bias(X, A_s, B_s, b1_s)
    O = tp.reduce_partials_bias(P, b2)
    if fused:
        D, dA, dB, dXp, db1, db2 = tp.mlp_bwd_bias(X, A_s, B_s, Z, Y, G)
    else:
        D, dA, dB, dXp = tp.mlp_bwd(X, A_s, B_s, Z, Y, G)
        db1 = tp.bias_grad(D)
        db2 = tp.bias_grad(G)
    dX = tp.reduce_partials(dXp)
    torch.cuda.synchronize()
    return dict(Z=Z, Y=Y, P=P, O=O, D=D, dA=dA, dB=dB, dXp=dXp, dX=dX, db1=db1, db2=db2)


def compare_biased(inp, bias, t, dtype, fused=False):
    X, A, B, G = (dev(inp[k]) for k in "XABG")
    b1, b2 = dev(bias["b1"]), dev(bias["b2"])
    n, d = X.shape
    m = A.shape[1]
    say(f"[gpu] biased step {dtype} n={n} d={d} m={m} t={t} fused={fused}")
    r = run_biased_step(X, shard_cols(A, t), shard_rows(B, t), b1.reshape(t, m // t).contiguous(), b2, G, fused)
    Xo, Ao, Bo, Go = (inp[k].f64 for k in "XABG")
    b1o, b2o = bias["b1"].f64, bias["b2"].f64
    fwd = om.tp_forward(Xo, Ao, Bo, t, b1=b1o, b2=b2o)
    bwd = om.tp_backward(Xo, Ao, Bo, fwd, Go)
    tol = TOL[dtype]
    errs = {"O": relerr(r["O"], fwd["O"]), "dX": relerr(r["dX"], bwd["dX"]),
            "db2": relerr(r["db2"], bwd["db2"])}
    for i in range(t):
        for k, ref in (("Z", fwd["Z"][i]), ("Y", fwd["Y"][i]), ("P", fwd["P"][i]), ("D", bwd["D"][i]),
                       ("dA", bwd["dA"][i]), ("dB", bwd["dB"][i]), ("dXp", bwd["dXp"][i]),
                       ("db1", bwd["db1"][i])):
            errs[f"{k}{i}"] = relerr(r[k][i], ref)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"over {tol}: {bad}"
    # the bias gradients are column sums of the stored D_i and of G: fp32 sums
    # of the given values, checked tighter
    for i in range(t):
        assert relerr(r["db1"][i], om.bias_grad(f64(r["D"][i]))) <= SUM_TOL
    assert relerr(r["db2"], om.bias_grad(Go)) <= SUM_TOL
    return errs


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("n,d,m,t", [(1, 4, 8, 2), (17, 36, 40, 2), (130, 72, 400, 2), (65, 100, 300, 3)])
def test_fp32_biased_ragged(n, d, m, t, fused):
    inp = mlp_inputs(n, d, m, t, dtype="f32", seed=21, x_std=1.0, w_std=0.2, g_std=1.0)
    compare_biased(inp, bias_inputs(m, d, "f32", seed=21), t, "f32", fused)


@pytest.mark.parametrize("n,d,m,t", [
    (1, 8, 16, 2),          # one token: one partial 128-row chunk
    (129, 264, 272, 2),     # a second chunk of one row; ragged N and K tails
    (1000, 264, 272, 2),    # ragged M inside a 256-row tile (chunk 7 of 8 is partial)
    (520, 520, 1584, 3),
    (300, 4096, 512, 2),    # a shape whose unbiased backward splits dgrad-1 (the fused one does not)
])
def test_bf16_fused_bias_grad(n, d, m, t):
    """tpmlp_bwd_bias against the oracle, and its D, dA, dB, dX_i against
    tpmlp_bwd's (the same products; bit for bit where tpmlp_bwd does not split
    dgrad-1), and its db1 against the column sums of its own stored D."""
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=22)
    bias = bias_inputs(m, d, "bf16", seed=22)
    compare_biased(inp, bias, t, "bf16", fused=True)
    X, A, B, G = (dev(inp[k]) for k in "XABG")
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    b1 = dev(bias["b1"]).reshape(t, m // t).contiguous()
    Z, Y, P = tp.mlp_fwd_bias(X, A_s, B_s, b1)
    f = tp.mlp_bwd_bias(X, A_s, B_s, Z, Y, G)
    u = tp.mlp_bwd(X, A_s, B_s, Z, Y, G)
    f2 = tp.mlp_bwd_bias(X, A_s, B_s, Z, Y, G)
    torch.cuda.synchronize()
    for a, b in zip(f, f2):  # repeatable bit for bit
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    if tp.bwd_workspace_bytes(X, A_s) == 0:
        for a, b in zip(f[:4], u):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("n,d,m,t", [
    (1, 8, 16, 2),
    (3, 264, 272, 2),
    (1000, 264, 272, 2),
    (520, 520, 1584, 3),
    (256, 256, 256, 1),
])
def test_bf16_biased_ragged(n, d, m, t):
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=6)
    compare_biased(inp, bias_inputs(m, d, "bf16", seed=6), t, "bf16")


def test_zero_bias_equals_unbiased_bitwise():
    """b1 = 0, b2 = 0: the biased launches give the unbiased ones' bits."""
    n, d, m, t = 300, 264, 528, 2
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=8)
    X, A, B = (dev(inp[k]) for k in "XAB")
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    Z0, Y0, P0 = tp.mlp_fwd(X, A_s, B_s)
    O0 = tp.reduce_partials(P0)
    Z1, Y1, P1 = tp.mlp_fwd_bias(X, A_s, B_s, torch.zeros((t, m // t), dtype=X.dtype, device="cuda"))
    O1 = tp.reduce_partials_bias(P1, torch.zeros(d, dtype=X.dtype, device="cuda"))
    torch.cuda.synchronize()
    for a, b in ((Z0, Z1), (Y0, Y1), (P0, P1), (O0, O1)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("t,rows,cols,dtype", [
    (1, 1, 1, "f32"),
    (3, 129, 5, "f32"),       # unaligned width: one column per thread
    (2, 300, 64, "bf16"),
    (8, 1000, 1544, "bf16"),  # ragged row chunk and column block
    (1, 8192, 3072, "bf16"),  # db2 of the 8.3B-shaped layer
    (2, 257, 24, "f32"),
])
def test_bias_grad_column_sums(t, rows, cols, dtype):
    g = mlp_inputs(rows, cols, 8, 1, dtype=dtype, seed=rows + cols, x_std=1.0)["X"]
    say(f"[gpu] bias_grad t={t} rows={rows} cols={cols} {dtype}")
    gd = dev(g).reshape(1, rows, cols).expand(t, rows, cols).contiguous()
    gd = gd * torch.arange(1, t + 1, dtype=gd.dtype, device="cuda").reshape(t, 1, 1)  # exact scalings
    db = tp.bias_grad(gd)
    db_again = tp.bias_grad(gd)
    torch.cuda.synchronize()
    ref = np.stack([om.bias_grad(f64(gd[i])) for i in range(t)])
    assert relerr(db, ref) <= SUM_TOL
    assert torch.equal(db, db_again)  # fixed summation order


def test_bias_grad_empty_rows_is_zero():
    g = torch.empty((2, 0, 16), dtype=torch.bfloat16, device="cuda")
    db = torch.full((2, 16), 7.0, dtype=torch.float32, device="cuda")
    tp.tpmlp_bias_grad(g, db)
    torch.cuda.synchronize()
    assert torch.count_nonzero(db) == 0


@pytest.mark.parametrize("t,rows,cols,in_dt,out_dt", [
    (3, 7, 5, "f32", "f32"),     # scalar path (cols % 8 != 0)
    (2, 33, 64, "bf16", "bf16"),
    (8, 100, 520, "bf16", "f32"),
    (4, 64, 24, "f32", "bf16"),
])
def test_reduce_partials_bias(t, rows, cols, in_dt, out_dt):
    parts = mlp_inputs(t * rows, cols, 8, 1, dtype=in_dt, seed=cols, x_std=1.0)["X"]
    b = bias_inputs(8, cols, out_dt, seed=cols)["b2"]
    pd = dev(parts).reshape(t, rows, cols).contiguous()
    out = tp.reduce_partials_bias(pd, dev(b))
    torch.cuda.synchronize()
    ref = om.reduce_partials([parts.f64.reshape(t, rows, cols)[i] for i in range(t)]) + b.f64[None, :]
    assert relerr(out, ref) <= TOL[out_dt]


# ------------------------------------------------------------------ full size, sampled
def test_gpt8p3b_biased_sampled():
    """h = 3072, m = 4h, t = 8, n = 8192 with both biases: sampled rows of the
    outputs and sampled hidden columns of the weight and bias gradients, each
    computed by the oracle one by one (rows and hidden units decompose)."""
    c = CONFIGS["gpt8p3b_t8"]
    t, m, d = c["t"], c["m"], c["d"]
    inp = config_inputs("gpt8p3b_t8", seed=0)
    bias = bias_inputs(m, d, "bf16", seed=0)
    X, A, B, G = (dev(inp[k]) for k in "XABG")
    b1, b2 = dev(bias["b1"]), dev(bias["b2"])
    say(f"[gpu] 8.3B-shaped biased step n={X.shape[0]} d={d} t={t}")
    r = run_biased_step(X, shard_cols(A, t), shard_rows(B, t), b1.reshape(t, m // t).contiguous(), b2, G)
    mi = m // t
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(X.shape[0], size=48, replace=False))
    Xf, Gf, Af, Bf = (inp[k].f32 for k in "XGAB")
    b1f, b2f = bias["b1"].f32, bias["b2"].f32
    errs = {}
    O_rows = np.zeros((rows.size, d))
    dX_rows = np.zeros((rows.size, d))
    for i in range(t):
        Ai, Bi, b1i = Af[:, i * mi:(i + 1) * mi], Bf[i * mi:(i + 1) * mi, :], b1f[i * mi:(i + 1) * mi]
        Z, Y, P = om.shard_forward(Xf[rows], Ai, Bi, b1_i=b1i)
        D, _, _, dXi = om.shard_backward(Xf[rows], Ai, Bi, Z, Y, Gf[rows])
        O_rows += P
        dX_rows += dXi
        for k, ref in (("Z", Z), ("Y", Y), ("P", P), ("D", D)):
            errs[f"{k}{i}[rows]"] = relerr(f64(r[k][i][rows]), ref)
        cols = np.sort(rng.choice(mi, size=32, replace=False))
        Zc, Yc, _ = om.shard_forward(Xf, Ai[:, cols], Bi[cols, :], b1_i=b1i[cols])
        Dc, dAc, dBc, _ = om.shard_backward(Xf, Ai[:, cols], Bi[cols, :], Zc, Yc, Gf)
        errs[f"dA{i}[:,H]"] = relerr(f64(r["dA"][i][:, cols]), dAc)
        errs[f"dB{i}[H,:]"] = relerr(f64(r["dB"][i][cols, :]), dBc)
        errs[f"db1_{i}[H]"] = relerr(f64(r["db1"][i][cols]), om.bias_grad(Dc))
    O_rows += b2f[None, :].astype(np.float64)
    errs["O[rows]"] = relerr(f64(r["O"][rows]), O_rows)
    errs["dX[rows]"] = relerr(f64(r["dX"][rows]), dX_rows)
    errs["db2"] = relerr(r["db2"], om.bias_grad(Gf))
    tol = TOL["bf16"]
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    say(f"[gpu] 8.3B-shaped biased: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"
    del r
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ sequence parallel
def run_sp_biased(inp, bias, t, p, seed, eps):
    x, A, B, G, gamma, beta = (dev(inp[k]) for k in ("x", "A", "B", "G", "gamma", "beta"))
    b1, b2 = dev(bias["b1"]), dev(bias["b2"])
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    m = A.shape[1]
    U, mean, rstd = tp.sp_ln_fwd(x, gamma, beta, t, eps)
    Z, Y, P = tp.mlp_fwd_bias(U, A_s, B_s, b1.reshape(t, m // t).contiguous())
    out = tp.sp_dropres_fwd(P, x, p, seed, bias=b2)
    dS = tp.sp_dropres_bwd(G, t, p, seed)
    D, dA, dB, dXp = tp.mlp_bwd(U, A_s, B_s, Z, Y, dS)
    db1 = tp.bias_grad(D)
    db2 = tp.bias_grad(dS)
    dx, dgamma, dbeta = tp.sp_ln_bwd(dXp, G, x, gamma, mean, rstd)
    torch.cuda.synchronize()
    return dict(out=out, dA=dA, dB=dB, dx=dx, dgamma=dgamma, dbeta=dbeta, db1=db1, db2=db2)


@pytest.mark.parametrize("s,h,m,t,dtype", [
    (64, 64, 256, 2, "f32"),
    (48, 24, 48, 4, "f32"),
    (96, 520, 1056, 4, "bf16"),
    (512, 4096, 2048, 8, "bf16"),
])
def test_sp_block_biased(s, h, m, t, dtype):
    inp = sp_inputs(s, h, m, t, dtype=dtype, seed=13)
    bias = bias_inputs(m, h, dtype, seed=13)
    p, seed, eps = 0.1, 4321, 1e-5
    say(f"[gpu] SP block with biases s={s} h={h} m={m} t={t} {dtype}")
    r = run_sp_biased(inp, bias, t, p, seed, eps)
    v = {k: inp[k].f64 for k in inp}
    b1o, b2o = bias["b1"].f64, bias["b2"].f64
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], eps, v["A"], v["B"], t, p, seed, b1=b1o, b2=b2o)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    tol = TOL[dtype]
    errs = {"out": relerr(r["out"], f["out"]), "dx": relerr(r["dx"], b["dx"]),
            "dgamma": relerr(r["dgamma"], b["dgamma"]), "dbeta": relerr(r["dbeta"], b["dbeta"]),
            "db2": relerr(r["db2"], b["mlp"]["db2"])}
    for i in range(t):
        errs[f"dA{i}"] = relerr(r["dA"][i], b["mlp"]["dA"][i])
        errs[f"dB{i}"] = relerr(r["dB"][i], b["mlp"]["dB"][i])
        errs[f"db1_{i}"] = relerr(r["db1"][i], b["mlp"]["db1"][i])
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] SP block with biases: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"
