"""Pins of the oracle's bias variants ([TRAIN] ColumnParallelLinear: the bias
is split like the output columns; RowParallelLinear: one unsplit bias added
after the all-reduce; custom autograd matmul rule: the bias gradient is the
upstream gradient summed over the rows; [EFF] §4.2: bias + GeLU and
bias + dropout + add).  Each check compares against something other than the
oracle's own formulas: torch's fp64 autograd, central finite differences, the
unsharded layer, a closed form, and the library's column sum."""

import numpy as np
import pytest
import torch

from oracle import mlp as om
from oracle import sp_block as osp
from tpmlp_inputs import mlp_inputs, sp_inputs


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _biases(seed, m, d, std=0.5):
    rng = np.random.default_rng(1000 + seed)
    return rng.standard_normal(m) * std, rng.standard_normal(d) * std


def _layer(seed=3, n=5, d=8, m=12, t=3):
    inp = mlp_inputs(n, d, m, t, dtype="f32", seed=seed, x_std=1.0, w_std=0.5, g_std=1.0)
    X, A, B, G = (inp[k].f64 for k in "XABG")
    b1, b2 = _biases(seed, m, d)
    return X, A, B, G, b1, b2


def check_torch_autograd(seed=3, n=5, d=8, m=12, t=3):
    """O = φ(X·A + b1)·B + b2 and all five gradients through torch's own fp64
    gelu and autograd."""
    X, A, B, G, b1, b2 = _layer(seed, n, d, m, t)
    tx, ta, tb, t1, t2 = (torch.tensor(v, requires_grad=True) for v in (X, A, B, b1, b2))
    O = torch.nn.functional.gelu(tx @ ta + t1, approximate="none") @ tb + t2
    (O * torch.tensor(G)).sum().backward()
    fwd = om.tp_forward(X, A, B, t, b1=b1, b2=b2)
    bwd = om.tp_backward(X, A, B, fwd, G)
    return bool(relerr(fwd["O"], O.detach().numpy()) < 1e-14
                and relerr(bwd["dX"], tx.grad.numpy()) < 1e-14
                and relerr(np.concatenate(bwd["dA"], 1), ta.grad.numpy()) < 1e-14
                and relerr(np.concatenate(bwd["dB"], 0), tb.grad.numpy()) < 1e-14
                and relerr(np.concatenate(bwd["db1"]), t1.grad.numpy()) < 1e-14
                and relerr(bwd["db2"], t2.grad.numpy()) < 1e-14)


def check_finite_differences(seed=5, n=3, d=4, m=8, t=2, step=1e-6):
    """Central differences of ℓ = Σ G⊙O on every entry of b1 and b2."""
    X, A, B, G, b1, b2 = _layer(seed, n, d, m, t)
    fwd = om.tp_forward(X, A, B, t, b1=b1, b2=b2)
    bwd = om.tp_backward(X, A, B, fwd, G)
    analytic = {"b1": np.concatenate(bwd["db1"]), "b2": bwd["db2"]}
    worst = 0.0
    for name in ("b1", "b2"):
        for k in range(analytic[name].shape[0]):
            vals = []
            for sgn in (1.0, -1.0):
                c1, c2 = b1.copy(), b2.copy()
                (c1 if name == "b1" else c2)[k] += sgn * step
                vals.append(om.loss(om.tp_forward(X, A, B, t, b1=c1, b2=c2)["O"], G))
            fd = (vals[0] - vals[1]) / (2 * step)
            worst = max(worst, abs(fd - analytic[name][k]) / max(1.0, abs(analytic[name][k])))
    return worst <= 1e-7


def check_sharded_equals_unsharded(seed=1, n=7, d=16, m=24, ts=(1, 2, 3, 4, 6, 24)):
    """Σ_i φ(X·A_i + b1_i)·B_i + b2 = φ(X·A + b1)·B + b2, and the gradient
    identities including hcat_i db1_i = db1, for every divisor t of m."""
    X, A, B, G, b1, b2 = _layer(seed, n, d, m, 1)
    O = om.dense_forward(X, A, B, b1=b1, b2=b2)
    dX, dA, dB, db1, db2 = om.dense_backward(X, A, B, G, b1=b1)
    ok = True
    for t in ts:
        fwd = om.tp_forward(X, A, B, t, b1=b1, b2=b2)
        bwd = om.tp_backward(X, A, B, fwd, G)
        ok &= relerr(fwd["O"], O) <= 1e-13
        ok &= relerr(bwd["dX"], dX) <= 1e-13
        ok &= relerr(np.concatenate(bwd["dA"], 1), dA) <= 1e-13
        ok &= relerr(np.concatenate(bwd["dB"], 0), dB) <= 1e-13
        ok &= relerr(np.concatenate(bwd["db1"]), db1) <= 1e-13
        ok &= relerr(bwd["db2"], db2) <= 1e-13
    return bool(ok)


def check_closed_form_zero_weights(seed=2, n=6, d=5, m=8, t=2):
    """With A = 0 every row of Z_i is b1_i: O = 1·(φ(b1)·B)ᵀ + b2 on every row,
    db2 = Σ_rows G, db1 = ((Σ_rows G)·Bᵀ) ⊙ φ'(b1), dA = Xᵀ·D with D's rows
    (G_r·Bᵀ) ⊙ φ'(b1) — all written out here without the oracle."""
    X, _, B, G, b1, b2 = _layer(seed, n, d, m, t)
    A = np.zeros((d, m))
    fwd = om.tp_forward(X, A, B, t, b1=b1, b2=b2)
    bwd = om.tp_backward(X, A, B, fwd, G)
    from scipy.special import erf
    phi = 0.5 * b1 * (1 + erf(b1 / np.sqrt(2)))
    dphi = 0.5 * (1 + erf(b1 / np.sqrt(2))) + b1 * np.exp(-0.5 * b1 ** 2) / np.sqrt(2 * np.pi)
    O = np.tile(phi @ B + b2, (n, 1))
    gsum = G.sum(axis=0)
    D = (G @ B.T) * dphi[None, :]
    return bool(relerr(fwd["O"], O) < 1e-14 and relerr(bwd["db2"], gsum) < 1e-14
                and relerr(np.concatenate(bwd["db1"]), (gsum @ B.T) * dphi) < 1e-13
                and relerr(np.concatenate(bwd["dA"], 1), X.T @ D) < 1e-13)


def check_zero_bias_is_no_bias(seed=4, n=5, d=8, m=12, t=3):
    """Zero biases give exactly the unbiased forward and backward."""
    X, A, B, G, _, _ = _layer(seed, n, d, m, t)
    f0 = om.tp_forward(X, A, B, t)
    fz = om.tp_forward(X, A, B, t, b1=np.zeros(m), b2=np.zeros(d))
    b0 = om.tp_backward(X, A, B, f0, G)
    bz = om.tp_backward(X, A, B, fz, G)
    return bool(np.array_equal(f0["O"], fz["O"]) and np.array_equal(b0["dX"], bz["dX"])
                and all(np.array_equal(p, q) for p, q in zip(b0["dA"], bz["dA"])))


def check_bias_grad_is_column_sum(seed=7):
    g = np.random.default_rng(seed).standard_normal((37, 11))
    return bool(relerr(om.bias_grad(g), g.sum(axis=0)) < 1e-14)


def check_sp_with_biases(seed=6, s=16, h=8, m=16, t=2, p=0.25, mask_seed=11):
    """The sequence-parallel block with biases (bias + dropout + add after the
    sum) against the dense block, forward and backward."""
    inp = sp_inputs(s, h, m, t, dtype="f32", seed=seed, x_std=1.0, w_std=0.4, g_std=1.0)
    v = {k: inp[k].f64 for k in ("x", "A", "B", "G", "gamma", "beta")}
    b1, b2 = _biases(seed, m, h)
    f = osp.sp_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], t, p, mask_seed, b1=b1, b2=b2)
    b = osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, p)
    df = osp.dense_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], p, mask_seed, b1=b1, b2=b2)
    db = osp.dense_backward(df, v["gamma"], v["A"], v["B"], v["G"], p, b1=b1)
    # the bias sits before the dropout: dropped elements lose their bias too
    M = df["mask"]
    S_plain = osp.dense_forward(v["x"], v["gamma"], v["beta"], 1e-5, v["A"], v["B"], p, mask_seed,
                                b1=b1)["out"] - v["x"]
    ok = relerr(f["out"], df["out"]) < 1e-13
    ok &= relerr(df["out"] - v["x"], S_plain + M * b2[None, :] / (1 - p)) < 1e-13
    ok &= relerr(b["dx"], db["dx"]) < 1e-12
    ok &= relerr(np.concatenate(b["mlp"]["db1"]), db["db1"]) < 1e-13
    ok &= relerr(b["mlp"]["db2"], db["db2"]) < 1e-13
    ok &= relerr(b["mlp"]["db2"], (v["G"] * M / (1 - p)).sum(axis=0)) < 1e-13
    return bool(ok)


BIAS_PINS = [check_torch_autograd, check_finite_differences, check_sharded_equals_unsharded,
             check_closed_form_zero_weights, check_zero_bias_is_no_bias, check_bias_grad_is_column_sum,
             check_sp_with_biases]


@pytest.mark.parametrize("pin", BIAS_PINS, ids=lambda f: f.__name__)
def test_bias_pin(pin):
    assert pin()


def _some_pin_fails():
    for p in BIAS_PINS:
        try:
            if not p():
                return True
        except Exception:
            return True
    return False


def test_mutant_row_bias_added_per_shard(monkeypatch):
    """Adding b2 to every partial (t times in total) is a plausible mistake."""
    orig = om.tp_forward

    def bad(X, A, B, t, act="gelu", b1=None, b2=None):
        out = orig(X, A, B, t, act, b1=b1, b2=b2)
        if b2 is not None:
            out["O"] = out["O"] + (t - 1) * np.asarray(b2)[None, :]
        return out
    monkeypatch.setattr(om, "tp_forward", bad)
    assert _some_pin_fails()


def test_mutant_column_bias_after_activation(monkeypatch):
    """Adding b1 after φ instead of before it."""
    orig = om.shard_forward

    def bad(X, A_i, B_i, act="gelu", b1_i=None):
        Z, Y, P = orig(X, A_i, B_i, act)
        if b1_i is not None:
            Y = Y + np.asarray(b1_i)[None, :]
            P = Y @ np.asarray(B_i, dtype=np.float64)
            Z = Z + np.asarray(b1_i)[None, :]
        return Z, Y, P
    monkeypatch.setattr(om, "shard_forward", bad)
    assert _some_pin_fails()


def test_mutant_bias_grad_mean_not_sum(monkeypatch):
    """A mean over the tokens instead of a sum."""
    monkeypatch.setattr(om, "bias_grad", lambda g: np.asarray(g, np.float64).mean(axis=0))
    assert _some_pin_fails()


def test_mutant_bias_grad_over_columns(monkeypatch):
    """Summing over the wrong axis (only shape-compatible when square)."""
    monkeypatch.setattr(om, "bias_grad", lambda g: np.asarray(g, np.float64).sum(axis=1)[: np.shape(g)[1]])
    assert _some_pin_fails()
