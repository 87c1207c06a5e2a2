"""Pins of the LayerNorm, Philox/dropout and sequence-parallel block oracles."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import layernorm as oln
from oracle import philox as oph
from oracle import sp_block as osp
from tpmlp_inputs import bf16_bits_to_f32, f32_to_bf16_bits, sp_inputs

from conftest import GOLDEN


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ------------------------------------------------------------------ checks
def check_philox_kat():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)["vectors"]
    for v in kat:
        c = [int(x, 16) for x in v["counter"]]
        k = [int(x, 16) for x in v["key"]]
        out = oph.philox4x32_10(*c, *k)
        if [int(o) for o in out] != [int(x, 16) for x in v["out"]]:
            return False
    return True


def check_ln_vs_torch(seed=0, rows=6, h=16, eps=1e-5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, h)) * 2 + 0.3
    gamma = 1 + 0.1 * rng.standard_normal(h)
    beta = 0.1 * rng.standard_normal(h)
    g = rng.standard_normal((rows, h))
    y, mean, rstd, xhat = oln.ln_forward(x, gamma, beta, eps)
    dx, dg, db = oln.ln_backward(g, xhat, rstd, gamma)
    tx, tg, tb = (torch.tensor(v, requires_grad=True) for v in (x, gamma, beta))
    ty = torch.nn.functional.layer_norm(tx, (h,), tg, tb, eps)
    (ty * torch.tensor(g)).sum().backward()
    return bool(relerr(y, ty.detach().numpy()) < 1e-14 and relerr(dx, tx.grad.numpy()) < 1e-13
                and relerr(dg, tg.grad.numpy()) < 1e-13 and relerr(db, tb.grad.numpy()) < 1e-14)


def check_ln_invariants(seed=1, rows=5, h=12, eps=1e-5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, h)) * 3 - 1
    gamma = np.ones(h)
    g = rng.standard_normal((rows, h))
    _, mean, rstd, xhat = oln.ln_forward(x, gamma, np.zeros(h), eps)
    var = x.var(axis=1)
    ok = np.max(np.abs(xhat.mean(axis=1))) < 1e-15 * h
    ok &= np.max(np.abs(xhat.var(axis=1) - var / (var + eps))) < 1e-14
    dx, _, _ = oln.ln_backward(g, xhat, rstd, gamma)
    # the input gradient has no component along 𝟏 ([TRAIN] LayerNorm section)
    ok &= np.max(np.abs(dx.sum(axis=1))) < 1e-13
    # along x̂ it keeps only the eps share: Σ dx·x̂ = rstd·(1 − mean(x̂²))·Σ g̃·x̂
    resid = rstd * (1 - (xhat ** 2).mean(axis=1)) * (g * xhat).sum(axis=1)
    ok &= np.max(np.abs((dx * xhat).sum(axis=1) - resid)) < 1e-13
    # with eps = 0 it is exactly orthogonal to x̂, as the page states
    _, _, rstd0, xhat0 = oln.ln_forward(x, gamma, np.zeros(h), 0.0)
    dx0, _, _ = oln.ln_backward(g, xhat0, rstd0, gamma)
    ok &= np.max(np.abs((dx0 * xhat0).sum(axis=1))) < 1e-13
    ok &= np.max(np.abs(dx0.sum(axis=1))) < 1e-13
    return bool(ok)


def _sp_tiny(seed=5, s=8, h=4, m=8, t=2):
    inp = sp_inputs(s, h, m, t, dtype="f32", seed=seed, x_std=1.0, w_std=0.5, g_std=1.0,
                    gamma_std=0.3, beta_std=0.3)
    return {k: v.f64 for k, v in inp.items()}


def check_sp_sharded_equals_dense(seed=7, s=16, h=8, m=16, t=4, p=0.25, mseed=11):
    v = _sp_tiny(seed, s, h, m, t)
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], t, p, mseed)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    fd = osp.dense_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], p, mseed)
    bd = osp.dense_backward(fd, v["gamma"], v["A"], v["B"], v["G"], p)
    ok = relerr(f["out"], fd["out"]) < 1e-14 and np.array_equal(f["mask"], fd["mask"])
    ok &= relerr(b["dx"], bd["dx"]) < 1e-13
    ok &= relerr(b["dgamma"], bd["dgamma"]) < 1e-13 and relerr(b["dbeta"], bd["dbeta"]) < 1e-13
    ok &= relerr(np.concatenate(b["mlp"]["dA"], 1), bd["dA"]) < 1e-13
    ok &= relerr(np.concatenate(b["mlp"]["dB"], 0), bd["dB"]) < 1e-13
    return bool(ok)


def check_sp_finite_differences(step=1e-6, p=0.25, mseed=3, t=2):
    v = _sp_tiny()
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], t, p, mseed)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    analytic = {"x": b["dx"], "gamma": b["dgamma"], "beta": b["dbeta"],
                "A": np.concatenate(b["mlp"]["dA"], 1), "B": np.concatenate(b["mlp"]["dB"], 0)}

    def L(vals):
        o = osp.sp_forward(vals["x"], vals["gamma"], vals["beta"], 1e-5, vals["A"], vals["B"], t, p, mseed)
        return float(np.sum(o["out"] * v["G"]))

    worst = 0.0
    for name in analytic:
        for idx in np.ndindex(v[name].shape):
            pv = {k: a.copy() for k, a in v.items()}
            mv = {k: a.copy() for k, a in v.items()}
            pv[name][idx] += step
            mv[name][idx] -= step
            fd = (L(pv) - L(mv)) / (2 * step)
            a = analytic[name][idx]
            worst = max(worst, abs(fd - a) / max(1.0, abs(a)))
    return worst <= 1e-7


def check_sp_vs_torch(p=0.25, mseed=9, t=2):
    v = _sp_tiny(seed=8, s=8, h=6, m=12)
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], t, p, mseed)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    tx, tg, tb, ta, tB = (torch.tensor(v[k], requires_grad=True) for k in ("x", "gamma", "beta", "A", "B"))
    u = torch.nn.functional.layer_norm(tx, (tx.shape[1],), tg, tb, 1e-5)
    S = torch.nn.functional.gelu(u @ ta, approximate="none") @ tB
    out = tx + torch.tensor(f["mask"].astype(np.float64)) * S / (1 - p)
    (out * torch.tensor(v["G"])).sum().backward()
    return bool(relerr(f["out"], out.detach().numpy()) < 1e-14
                and relerr(b["dx"], tx.grad.numpy()) < 1e-13
                and relerr(b["dgamma"], tg.grad.numpy()) < 1e-13
                and relerr(b["dbeta"], tb.grad.numpy()) < 1e-13)


# ------------------------------------------------------------------ tests
def test_philox_known_answers():
    assert check_philox_kat()


def test_keep_fraction_and_scale():
    # 2^22 draws, p = 0.1: the kept fraction lies within 6σ of 0.9
    h = 4096
    M = oph.keep_mask(0, 1024, h, 0.1, seed=0)
    frac = M.mean()
    sigma = np.sqrt(0.9 * 0.1 / M.size)
    assert abs(frac - 0.9) < 6 * sigma
    assert oph.drop_threshold(0.1) == 429496729
    assert oph.drop_threshold(0.0) == 0


def test_masks_differ_between_sequence_shards():
    # each SP rank must draw its own mask ([SP] RNG-domain table; Megatron issue #1256)
    s, h, t = 4096, 4096, 8
    sl = s // t
    masks = [oph.keep_mask(r * sl, 8, h, 0.1, seed=0) for r in range(t)]  # first 8 rows of each shard
    for i in range(t):
        for j in range(i + 1, t):
            assert not np.array_equal(masks[i], masks[j])


def test_mask_is_keyed_by_global_index():
    full = oph.keep_mask(0, 64, 40, 0.3, seed=12345678901)
    part = oph.keep_mask(17, 9, 40, 0.3, seed=12345678901)
    assert np.array_equal(full[17:26], part)
    assert not np.array_equal(oph.keep_mask(0, 64, 40, 0.3, seed=1), full)


def test_layernorm_matches_torch():
    assert check_ln_vs_torch()


def test_layernorm_invariants():
    assert check_ln_invariants()


def test_sp_sharded_equals_dense():
    assert check_sp_sharded_equals_dense()


def test_sp_finite_differences():
    assert check_sp_finite_differences()


def test_sp_matches_torch():
    assert check_sp_vs_torch()


def test_sp_requires_t_at_least_2():
    v = _sp_tiny()
    with pytest.raises(ValueError):
        osp.sp_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], 1, 0.1, 0)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
