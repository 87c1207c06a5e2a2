"""Pins of the vocabulary-parallel cross-entropy oracle (oracle/vocab_ce.py):
torch's fp64 cross_entropy and its autograd, the split statistics against the
unsplit log-sum-exp for every divisor t, central finite differences, the
closed form of all-zero logits, and planted mistakes that must fail a pin."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import vocab_ce as ov
from tpmlp_inputs import vocab_inputs


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _case(n=7, h=6, V=24, seed=0, w_std=0.7):
    inp = vocab_inputs(n, h, V, dtype="f32", seed=seed, x_std=1.0, w_std=w_std, g_std=1.0)
    return inp["X"].f64, inp["W"].f64, inp["targets"], inp["g"].f64


def check_torch_cross_entropy(t=3):
    X, W, tg, g = _case()
    tX, tW = torch.tensor(X, requires_grad=True), torch.tensor(W, requires_grad=True)
    loss = F.cross_entropy(tX @ tW.T, torch.tensor(tg, dtype=torch.long), reduction="none")
    (loss * torch.tensor(g)).sum().backward()
    f = ov.tp_forward(X, W, tg, t)
    b = ov.tp_backward(X, W, tg, f, g)
    return bool(relerr(f["loss"], loss.detach().numpy()) < 1e-13 and relerr(b["dX"], tX.grad.numpy()) < 1e-12
                and relerr(np.concatenate(b["dW"], 0), tW.grad.numpy()) < 1e-12)


def check_split_equals_unsplit():
    """Eq. (3)/(4): the combined shard statistics give logsumexp − target of the
    whole row for every t dividing V, and the combined max is the row max."""
    X, W, tg, _ = _case(V=24)
    ref = ov.dense_loss(X, W, tg)
    L = X @ W.T
    ok = True
    for t in (1, 2, 3, 4, 6, 8, 12, 24):
        f = ov.tp_forward(X, W, tg, t)
        ok &= relerr(f["loss"], ref) < 1e-13
        ok &= np.allclose(f["max"], L.max(axis=1), rtol=1e-14, atol=0)  # per-shard products round alike to 1 ulp
    return bool(ok)


def check_finite_differences(step=1e-6):
    X, W, tg, g = _case(n=3, h=4, V=6, seed=2)
    t = 2
    f = ov.tp_forward(X, W, tg, t)
    b = ov.tp_backward(X, W, tg, f, g)
    grads = {"X": b["dX"], "W": np.concatenate(b["dW"], 0)}
    worst = 0.0
    for name in ("X", "W"):
        for idx in np.ndindex(grads[name].shape):
            vals = []
            for sgn in (1.0, -1.0):
                Xc, Wc = X.copy(), W.copy()
                (Xc if name == "X" else Wc)[idx] += sgn * step
                vals.append(float((ov.tp_forward(Xc, Wc, tg, t)["loss"] * g).sum()))
            fd = (vals[0] - vals[1]) / (2 * step)
            worst = max(worst, abs(fd - grads[name][idx]) / max(1.0, abs(grads[name][idx])))
    return worst <= 1e-7


def check_zero_logits_closed_form():
    """W = 0: every logit is 0, the loss is ln V for every token, and
    dlogits = g·(1/V − onehot)."""
    X, W, tg, g = _case(V=24)
    W = np.zeros_like(W)
    f = ov.tp_forward(X, W, tg, 4)
    b = ov.tp_backward(X, W, tg, f, g)
    n, V = X.shape[0], W.shape[0]
    D = np.full((n, V), 1.0 / V)
    D[np.arange(n), tg] -= 1.0
    D *= g[:, None]
    return bool(np.allclose(f["loss"], np.log(V), rtol=0, atol=1e-14)
                and relerr(np.concatenate(b["dlogits"], 1), D) < 1e-14)


def check_gradient_rows_sum_to_zero():
    """Σ_k dlogits[r, k] = g_r·(1 − 1) = 0 on every row."""
    X, W, tg, g = _case()
    f = ov.tp_forward(X, W, tg, 3)
    b = ov.tp_backward(X, W, tg, f, g)
    return bool(np.abs(np.concatenate(b["dlogits"], 1).sum(axis=1)).max() < 1e-13)


PINS = [check_torch_cross_entropy, check_split_equals_unsplit, check_finite_differences,
        check_zero_logits_closed_form, check_gradient_rows_sum_to_zero]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_vocab_ce_pin(pin):
    assert pin()


def _some_pin_fails():
    for p in PINS:
        try:
            if not p():
                return True
        except Exception:
            return True
    return False


def test_mutant_sum_without_rescale(monkeypatch):
    """Adding the shards' s_i without the exp(m_i − m) factor."""
    def bad(stats):
        m = np.max(np.stack([st[0] for st in stats]), axis=0)
        S = sum(st[1] for st in stats)
        tau = sum(st[2] for st in stats)
        return m, S, np.log(S) + m - tau
    monkeypatch.setattr(ov, "combine", bad)
    assert _some_pin_fails()


def test_mutant_target_in_every_shard(monkeypatch):
    """Every shard contributing a target logit (wrong offset: local index)."""
    def bad(logits_i, targets, start):
        L = np.asarray(logits_i, np.float64)
        m = L.max(axis=1)
        s = np.exp(L - m[:, None]).sum(axis=1)
        tau = np.array([L[r, int(targets[r]) % L.shape[1]] for r in range(L.shape[0])])
        return m, s, tau
    monkeypatch.setattr(ov, "shard_stats", bad)
    assert _some_pin_fails()


def test_mutant_mean_instead_of_max(monkeypatch):
    """The first reduction taken as a mean (the stabiliser must be the max for
    the closed forms; with the rescale the value survives, so this checks the
    pins see the combined max)."""
    def bad(stats):
        m = np.mean(np.stack([st[0] for st in stats]), axis=0)
        S = sum(st[1] * np.exp(st[0] - m) for st in stats)
        tau = sum(st[2] for st in stats)
        return m, S, np.log(S) + m - tau
    monkeypatch.setattr(ov, "combine", bad)
    assert _some_pin_fails()
