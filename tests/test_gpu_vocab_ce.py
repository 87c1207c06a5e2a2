"""GPU parity of the vocabulary-parallel logit layer and cross-entropy
(tpmlp_vocab_ce_fwd / _bwd) against the fp64 oracle (oracle/vocab_ce.py) on the
same seeded inputs, through the C ABI.

Bars (relative Frobenius error, fp64): fp32 path 1e-5, bf16 path 8e-3, for the
logits, the loss, the row maximum and log-normaliser, dlogits, dW and dX.  The oracle takes the rounded inputs upcast exactly; on the bf16 path the
GPU's statistics come from its bf16-rounded logits, which the bar absorbs.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import vocab_ce as ov
from tpmlp_inputs import CONFIGS, config_inputs, vocab_inputs

from gpu_util import dev, f64, relerr, say

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3}


def lse(rmax, rsum):
    """The row's log-normaliser ln Σ exp(x) = ln(row_sum) + row_max.  It is
    compared rather than row_sum alone, whose scale exp(−row_max) moves with
    the bf16 rounding of the largest logit (the product does not)."""
    return np.log(f64(rsum)) + f64(rmax)


def shard_vocab(W, t):
    V, h = W.shape
    return W.reshape(t, V // t, h).contiguous()


def run(inp, t, vocab_start=0):
    X, W = dev(inp["X"]), dev(inp["W"])
    tg = torch.from_numpy(inp["targets"]).cuda()
    g = torch.from_numpy(inp["g"].f32.copy()).cuda()
    Ws = shard_vocab(W, t) if W.shape[0] % t == 0 else None
    logits, loss, rmax, rsum = tp.vocab_ce_fwd(X, Ws, tg, vocab_start)
    dlogits, dW, dXp = tp.vocab_ce_bwd(X, Ws, tg, logits, rmax, rsum, g, vocab_start)
    dX = tp.reduce_partials(dXp)
    torch.cuda.synchronize()
    return dict(logits=logits, loss=loss, rmax=rmax, rsum=rsum, dlogits=dlogits, dW=dW, dX=dX)


def compare(n, h, V, t, dtype, seed=0):
    # weights of std 1.2/√h give logits of std ≈ 1.2, as the 0.02 initialisation
    # gives at h = 3072; much larger logits make the bf16 rounding of the row
    # maximum dominate the normaliser
    say(f"[gpu] vocab CE {dtype} n={n} h={h} V={V} t={t}")
    inp = vocab_inputs(n, h, V, dtype=dtype, seed=seed, x_std=1.0, w_std=1.2 / np.sqrt(h), g_std=1.0)
    r = run(inp, t)
    X, W, tg, g = inp["X"].f64, inp["W"].f64, inp["targets"], inp["g"].f64
    f = ov.tp_forward(X, W, tg, t)
    b = ov.tp_backward(X, W, tg, f, g)
    errs = {"loss": relerr(r["loss"], f["loss"]), "rmax": relerr(r["rmax"], f["max"]),
            "lse": relerr(lse(r["rmax"], r["rsum"]), np.log(f["sum"]) + f["max"]), "dX": relerr(r["dX"], b["dX"])}
    for i in range(t):
        errs[f"logits{i}"] = relerr(r["logits"][i], f["logits"][i])
        errs[f"dlogits{i}"] = relerr(r["dlogits"][i], b["dlogits"][i])
        errs[f"dW{i}"] = relerr(r["dW"][i], b["dW"][i])
    tol = TOL[dtype]
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] vocab CE: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"


@pytest.mark.parametrize("n,h,V,t", [(1, 4, 6, 2), (7, 6, 24, 3), (33, 20, 30, 3), (130, 72, 400, 4)])
def test_fp32(n, h, V, t):
    compare(n, h, V, t, "f32")


@pytest.mark.parametrize("n,h,V,t", [(1, 8, 16, 2), (37, 64, 320, 4), (300, 264, 2064, 2), (520, 520, 1056, 1)])
def test_bf16(n, h, V, t):
    compare(n, h, V, t, "bf16")


def test_one_shard_of_many_is_the_rank_partial():
    """t_local = 1 holding shard 2 of 4 (vocab_start = 2·v_i): the returned row
    statistics are that shard's own (m_i, s_i) and the loss ln s_i + m_i − τ_i,
    the rank's inputs to the three all-reduces; targets of other shards give
    τ_i = 0."""
    n, h, V, t = 50, 64, 256, 4
    inp = vocab_inputs(n, h, V, dtype="bf16", seed=3, x_std=1.0, w_std=1.2 / np.sqrt(h))
    vi = V // t
    X = dev(inp["X"])
    W2 = dev(inp["W"])[2 * vi:3 * vi].reshape(1, vi, h).contiguous()
    tg = torch.from_numpy(inp["targets"]).cuda()
    logits, loss, rmax, rsum = tp.vocab_ce_fwd(X, W2, tg, vocab_start=2 * vi)
    torch.cuda.synchronize()
    L2 = ov.shard_logits(inp["X"].f64, inp["W"].f64[2 * vi:3 * vi])
    m, s, tau = ov.shard_stats(L2, inp["targets"], 2 * vi)
    assert relerr(rmax, m) <= TOL["bf16"] and relerr(lse(rmax, rsum), np.log(s) + m) <= TOL["bf16"]
    assert relerr(loss, np.log(s) + m - tau) <= TOL["bf16"]
    own = (inp["targets"] >= 2 * vi) & (inp["targets"] < 3 * vi)
    assert 0 < own.sum() < n  # both kinds of token are present


def test_deterministic_bitwise():
    inp = vocab_inputs(200, 64, 512, dtype="bf16", seed=5, x_std=1.0, w_std=0.15)
    r1, r2 = run(inp, 4), run(inp, 4)
    for k in r1:
        a, b = r1[k], r2[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k


def test_gpt8p3b_vocab_sampled():
    """n = 8192 tokens, h = 3072, V = 51200 in t = 8 shards of 6400, g = 1/n (the
    mean loss): sampled tokens' logits, loss, row statistics, dlogits and dX
    rows computed by the oracle one token at a time (a token's row depends only
    on its own X row and target)."""
    c = CONFIGS["gpt8p3b_vocab_t8"]
    n, h, V, t = c["n"], c["d"], c["V"], c["t"]
    inp = config_inputs("gpt8p3b_vocab_t8", seed=0)
    say(f"[gpu] 8.3B-shaped vocab CE: n={n} h={h} V={V} t={t}")
    r = run(inp, t)
    rows = np.sort(np.random.default_rng(4).choice(n, size=48, replace=False))
    X, W, tg, g = inp["X"].f32[rows], inp["W"].f32, inp["targets"][rows], inp["g"].f64[rows]
    f = ov.tp_forward(X, W, tg, t)
    b = ov.tp_backward(X, W, tg, f, g)
    errs = {"loss": relerr(f64(r["loss"])[rows], f["loss"]), "rmax": relerr(f64(r["rmax"])[rows], f["max"]),
            "lse": relerr(lse(r["rmax"], r["rsum"])[rows], np.log(f["sum"]) + f["max"]),
            "dX": relerr(f64(r["dX"])[rows], b["dX"])}
    for i in range(t):
        errs[f"logits{i}"] = relerr(f64(r["logits"][i])[rows], f["logits"][i])
        errs[f"dlogits{i}"] = relerr(f64(r["dlogits"][i])[rows], b["dlogits"][i])
    bad = {k: e for k, e in errs.items() if not (e <= TOL["bf16"])}
    say(f"[gpu] 8.3B-shaped vocab CE: worst {max(errs.values()):.3e}")
    assert not bad, f"over {TOL['bf16']}: {bad}"
    del r
    torch.cuda.empty_cache()
