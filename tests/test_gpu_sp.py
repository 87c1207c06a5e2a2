"""GPU parity of the sequence-parallel region (tpmlp_ln_sp) together with the
MLP shards, against the fp64 oracle's sharded SP block on the same inputs."""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import philox as oph
from oracle import sp_block as osp
from tpmlp_inputs import CONFIGS, config_inputs, sp_inputs

from gpu_util import dev, f64, relerr, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3}


def run_block(inp, t, p, seed, eps):
    x, A, B, G, gamma, beta = (dev(inp[k]) for k in ("x", "A", "B", "G", "gamma", "beta"))
    A_s, B_s = shard_cols(A, t), shard_rows(B, t)
    U, mean, rstd = tp.sp_ln_fwd(x, gamma, beta, t, eps)
    Z, Y, P = tp.mlp_fwd(U, A_s, B_s)
    out = tp.sp_dropres_fwd(P, x, p, seed)
    dS = tp.sp_dropres_bwd(G, t, p, seed)
    D, dA, dB, dXp = tp.mlp_bwd(U, A_s, B_s, Z, Y, dS)
    dx, dgamma, dbeta = tp.sp_ln_bwd(dXp, G, x, gamma, mean, rstd)
    torch.cuda.synchronize()
    return dict(U=U, mean=mean, rstd=rstd, out=out, dS=dS, dA=dA, dB=dB, dx=dx,
                dgamma=dgamma, dbeta=dbeta)


def check_block(inp, t, p, seed, eps, dtype, label):
    s, h = inp["x"].shape
    say(f"[gpu] SP block {label}: s={s} h={h} t={t} {dtype}")
    r = run_block(inp, t, p, seed, eps)
    v = {k: inp[k].f64 for k in inp}
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], eps, v["A"], v["B"], t, p, seed)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    # the keep-mask is integer work: bit-exact
    gpu_mask = f64(r["dS"]) != 0.0
    ref_mask = f["mask"] & (v["G"] != 0.0)
    assert np.array_equal(gpu_mask, ref_mask), "dropout mask differs from the oracle"
    tol = TOL[dtype]
    errs = {"U": relerr(r["U"], f["U"]), "out": relerr(r["out"], f["out"]),
            "dx": relerr(r["dx"], b["dx"]), "dgamma": relerr(r["dgamma"], b["dgamma"]),
            "dbeta": relerr(r["dbeta"], b["dbeta"]), "mean": relerr(r["mean"], f["mean"]),
            "rstd": relerr(r["rstd"], f["rstd"])}
    for i in range(t):
        errs[f"dA{i}"] = relerr(r["dA"][i], b["mlp"]["dA"][i])
        errs[f"dB{i}"] = relerr(r["dB"][i], b["mlp"]["dB"][i])
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] SP block {label}: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"


@pytest.mark.parametrize("s,h,m,t,dtype", [
    (64, 64, 256, 2, "f32"),
    (48, 24, 48, 4, "f32"),
    (96, 520, 1056, 4, "bf16"),
    (512, 4096, 2048, 8, "bf16"),
    # rows wider than 4096 (the GPT-1T-shaped layer's h = 25600): the LN
    # kernels loop over 4096-element pieces of a row
    (64, 6144, 512, 2, "bf16"),
    (32, 25600, 256, 2, "bf16"),
    (16, 4104, 64, 2, "f32"),
    (24, 6144, 96, 4, "f32"),
])
def test_sp_block_small(s, h, m, t, dtype):
    inp = sp_inputs(s, h, m, t, dtype=dtype, seed=3)
    check_block(inp, t, 0.1, 1234, 1e-5, dtype, "small")


def test_sp_block_config():
    """s = 4096, h = 4096, m = 4h, t = 8, p = 0.1, eps = 1e-5: full comparison."""
    c = CONFIGS["sp_block_t8"]
    check_block(config_inputs("sp_block_t8", seed=0), c["t"], c["p"], c["mask_seed"], c["eps"],
                "bf16", "config")


def test_dropout_row_offset_and_zero_p():
    s, h, t = 64, 128, 2
    g = torch.ones((s, h), dtype=torch.bfloat16, device="cuda")
    d0 = tp.sp_dropres_bwd(g, t, 0.3, seed=77, row0=5)
    torch.cuda.synchronize()
    assert np.array_equal(f64(d0) != 0, oph.keep_mask(5, s, h, 0.3, seed=77))
    kept = f64(d0)[f64(d0) != 0]
    assert np.allclose(kept, 1.0 / 0.7, rtol=4e-3)  # bf16-rounded 1/(1-p)
    d1 = tp.sp_dropres_bwd(g, t, 0.0, seed=77)
    torch.cuda.synchronize()
    assert torch.equal(d1, g)
