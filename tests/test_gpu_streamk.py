"""K-split tail of the bf16 GEMMs (tpmlp_set_gemm_tile_policy(GEMM_STREAMK)).

A launch of one problem whose 256×256 tiles fill whole rounds of the 256 CUs
and at most half of one more runs each leftover tile as q equal K pieces of
fp32 partials (q·tiles ≤ 256, one extra round), added per tile in K order
by a fix-up kernel that applies the epilogue.  Checked here: parity with the
fp64 oracle, the same bits on every run, and agreement with plain 256×256
tiles to bf16 rounding (the tail tiles' K sums are added in pieces, a
different fp32 rounding).  Shapes: 16 tail tiles in 4 pieces of one K step
(also with ragged M, N and a ragged last K step) and 100 tail tiles in 2
pieces of 5 steps.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import mlp as om
from tpmlp_inputs import bias_inputs, mlp_inputs

from gpu_util import dev, relerr, run_step, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def restore_policy():
    yield
    tp.set_gemm_tile_policy(tp.GEMM_TILE_AUTO)


def bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def step(inp, t, policy):
    tp.set_gemm_tile_policy(policy)
    X, A, B, G = (dev(inp[k]) for k in "XABG")
    return run_step(X, shard_cols(A, t), shard_rows(B, t), G)


@pytest.mark.parametrize("n,d,m,t", [
    # GEMM1 and dgrad-1: 17 × 16 = 272 tiles (one round + 16), K = 256: four
    # pieces of one K step per tail tile
    (4352, 256, 4096, 1),
    # ragged: 4300 rows, K = 200 (the last step 8 wide), N = 4000
    (4300, 200, 4000, 1),
    # 4 × 89 = 356 tiles (one round + 100), K = 640 (10 steps): two pieces
    # of 5 steps per tail tile
    (1024, 640, 22784, 1),
])
def test_stream_k_tail(n, d, m, t):
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=41)
    say(f"[gpu] stream-K n={n} d={d} m={m} t={t}")
    sk = step(inp, t, tp.GEMM_STREAMK)
    sk2 = step(inp, t, tp.GEMM_STREAMK)
    plain = step(inp, t, tp.GEMM_TILE_256)
    for k in sk:
        assert torch.equal(bits(sk[k]), bits(sk2[k])), f"{k}: not reproducible"
        e = relerr(sk[k], plain[k].float().cpu().numpy().astype(np.float64))
        assert e <= 2e-3, f"{k}: stream-K vs whole tiles {e:.2e}"
    Xo, Ao, Bo, Go = (inp[k].f64 for k in "XABG")
    fwd = om.tp_forward(Xo, Ao, Bo, t)
    bwd = om.tp_backward(Xo, Ao, Bo, fwd, Go)
    errs = {"O": relerr(sk["O"], fwd["O"]), "dX": relerr(sk["dX"], bwd["dX"])}
    for i in range(t):
        for k, ref in (("Z", fwd["Z"][i]), ("Y", fwd["Y"][i]), ("P", fwd["P"][i]), ("D", bwd["D"][i]),
                       ("dA", bwd["dA"][i]), ("dB", bwd["dB"][i]), ("dXp", bwd["dXp"][i])):
            errs[f"{k}{i}"] = relerr(sk[k][i], ref)
    say(f"[gpu] stream-K: worst {max(errs.values()):.3e} ({max(errs, key=errs.get)})")
    assert max(errs.values()) <= 8e-3, errs


def test_stream_k_biased_forward():
    """Z = X·A_i + b1, Y = GeLU(Z) with the bias added in the fix-up."""
    n, d, m, t = 4352, 256, 4096, 1
    inp = mlp_inputs(n, d, m, t, dtype="bf16", seed=42)
    bias = bias_inputs(m, d, "bf16", seed=42)
    X, A, B = (dev(inp[k]) for k in "XAB")
    b1 = dev(bias["b1"]).reshape(t, m // t).contiguous()
    tp.set_gemm_tile_policy(tp.GEMM_STREAMK)
    Z, Y, P = tp.mlp_fwd_bias(X, shard_cols(A, t), shard_rows(B, t), b1)
    torch.cuda.synchronize()
    fwd = om.tp_forward(inp["X"].f64, inp["A"].f64, inp["B"].f64, t, b1=bias["b1"].f64)
    assert relerr(Z[0], fwd["Z"][0]) <= 8e-3
    assert relerr(Y[0], fwd["Y"][0]) <= 8e-3
    assert relerr(P[0], fwd["P"][0]) <= 8e-3
