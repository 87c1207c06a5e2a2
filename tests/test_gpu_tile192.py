"""The bf16 GEMMs' narrow output tiles, 256×192 and 256×128
(tpmlp_set_gemm_tile_policy).

Each output element's K sum runs in the same order with either tile width,
so every result must equal the 256×256 tiles' bit for bit; the small shapes
are also compared with the fp64 oracle.  Shapes have ragged edges in every
dimension (M not a multiple of 256, N not a multiple of 192 or 128, K not a
multiple of 64) and include one shard of the 8.3B-shaped layer (n = 8192,
d = 3072, m_i = 1536), where the automatic policy picks 256×192 for the
forward GEMMs and dgrad-1, and the single-shard layer (n = 2048, d = 1024,
m = 4096), where it picks 256×128 for Z = X·A and dgrad-1.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import attention as oa
from oracle import mlp as om
from tpmlp_inputs import attn_inputs, bias_inputs, mlp_inputs

from gpu_util import dev, relerr, run_step, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu

POLICIES = (tp.GEMM_TILE_256, tp.GEMM_TILE_192, tp.GEMM_TILE_128, tp.GEMM_TILE_AUTO)


@pytest.fixture(autouse=True)
def restore_policy():
    yield
    tp.set_gemm_tile_policy(tp.GEMM_TILE_AUTO)


def bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def same_bits(a, b, name):
    assert a.shape == b.shape, name
    eq = torch.equal(bits(a), bits(b))
    if not eq:
        diff = (a.float() - b.float()).abs()
        idx = int(torch.argmax(diff))
        pytest.fail(f"{name}: results differ between tile widths, max |Δ| {float(diff.max()):.3e} at flat {idx}")


@pytest.mark.parametrize("n,d,m,t", [
    (300, 264, 528, 2),      # N of GEMM1 = 264: one full and one 72-wide tile of 192
    (520, 392, 776, 1),      # K = 392 (6 steps + 8), N = 776 and 392
    (17, 1000, 2000, 2),     # a single ragged row block, K = 1000
    (8192, 3072, 1536, 1),   # one shard of the 8.3B-shaped layer (256x192 tiles chosen)
    (2048, 1024, 4096, 1),   # the single-shard layer (256x128 tiles chosen for GEMM1 and dgrad-1)
])
def test_step_is_bit_identical_across_tile_widths(n, d, m, t):
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=31)
    X, A, B, G = (dev(inp[k]) for k in "XABG")
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    runs = {}
    for p in POLICIES:
        tp.set_gemm_tile_policy(p)
        say(f"[gpu] tile policy {p}: n={n} d={d} m={m} t={t}")
        runs[p] = run_step(X, A_s, B_s, G)
    for p in POLICIES[1:]:
        for k in runs[POLICIES[0]]:
            same_bits(runs[POLICIES[0]][k], runs[p][k], f"{k} (policy {p})")
    if n * d * m <= 1 << 28:
        Xo, Ao, Bo, Go = (inp[k].f64 for k in "XABG")
        fwd = om.tp_forward(Xo, Ao, Bo, t)
        bwd = om.tp_backward(Xo, Ao, Bo, fwd, Go)
        r = runs[tp.GEMM_TILE_192]
        errs = {"O": relerr(r["O"], fwd["O"]), "dX": relerr(r["dX"], bwd["dX"])}
        for i in range(t):
            for k, ref in (("Z", fwd["Z"][i]), ("Y", fwd["Y"][i]), ("P", fwd["P"][i]), ("D", bwd["D"][i]),
                           ("dA", bwd["dA"][i]), ("dB", bwd["dB"][i])):
                errs[f"{k}{i}"] = relerr(r[k][i], ref)
        say(f"[gpu] 256x192 tiles: worst {max(errs.values()):.3e} ({max(errs, key=errs.get)})")
        assert max(errs.values()) <= 8e-3, errs
    del runs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,d,m,t", [(300, 264, 528, 2), (257, 392, 1160, 1)])
def test_biased_forward_is_bit_identical_across_tile_widths(n, d, m, t):
    """The bias + GeLU epilogue (Z and Y in two passes) on 256×192 tiles."""
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=32)
    bias = bias_inputs(m, d, "bf16", seed=32)
    X, A, B = (dev(inp[k]) for k in "XAB")
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    b1 = dev(bias["b1"]).reshape(t, m // t).contiguous()
    out = {}
    for p in POLICIES[:3]:
        tp.set_gemm_tile_policy(p)
        out[p] = tp.mlp_fwd_bias(X, A_s, B_s, b1)
        torch.cuda.synchronize()
    for p in POLICIES[1:3]:
        for name, a, b in zip("ZYP", out[POLICIES[0]], out[p]):
            same_bits(a, b, f"{name} (policy {p})")
    fwd = om.tp_forward(inp["X"].f64, inp["A"].f64, inp["B"].f64, t, b1=bias["b1"].f64)
    Z, Y, P = out[tp.GEMM_TILE_192]
    for i in range(t):
        assert relerr(Z[i], fwd["Z"][i]) <= 8e-3
        assert relerr(Y[i], fwd["Y"][i]) <= 8e-3
        assert relerr(P[i], fwd["P"][i]) <= 8e-3


@pytest.mark.parametrize("bias", [False, True])
def test_attention_layer_is_bit_identical_across_tile_widths(bias):
    """QKV (N = 3w = 1152 per shard at the 8.3B shape; here 3·256/2 = 384,
    two 192-wide tiles) with the plain or bias epilogue, and the projection."""
    s, b, d, heads, t = 70, 3, 256, 4, 2
    inp = attn_inputs(s, b, d, heads, dtype="bf16", seed=33, x_std=1.0, w_std=1.2 / np.sqrt(d), g_std=1.0,
                      bias_std=0.5)
    X, Wq, Wp = (dev(inp[k]) for k in ("X", "Wqkv", "Wproj"))
    Wq_s, Wp_s = shard_cols(Wq, t), shard_rows(Wp, t)
    bq = dev(inp["bqkv"]).reshape(t, 3 * d // t).contiguous() if bias else None
    out = {}
    for p in POLICIES[:3]:
        tp.set_gemm_tile_policy(p)
        out[p] = tp.attn_fwd(X, Wq_s, Wp_s, s, b, d // heads, True, bqkv=bq)
        torch.cuda.synchronize()
    for p in POLICIES[1:3]:
        for name, a, c in zip(("QKV", "O", "lse", "P"), out[POLICIES[0]], out[p]):
            same_bits(a, c, f"{name} (policy {p})")
    L = {k: v.f64 for k, v in inp.items()}
    f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, True,
                      bqkv=L["bqkv"] if bias else None)
    QKV, O, lse, P = out[tp.GEMM_TILE_192]
    for i in range(t):
        assert relerr(QKV[i], f["shards"][i]["QKV"]) <= 8e-3
        assert relerr(P[i], f["shards"][i]["P"]) <= 8e-3
