"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each.  This is what makes the pins worth trusting: a pin that
a dropped term, a wrong sign, a transposed operand or a wrong split axis slips
through is no pin."""

import numpy as np
import pytest
from scipy.special import erf

import test_oracle_mlp as M
import test_oracle_sp as S
from oracle import layernorm as oln
from oracle import mlp as om
from oracle import philox as oph

MLP_PINS = [M.check_gelu_table, M.check_gelu_identities, M.check_gelu_vs_torch,
            M.check_finite_differences, M.check_torch_autograd,
            M.check_sharded_equals_unsharded, M.check_bruteforce_loops]
SP_PINS = [S.check_ln_vs_torch, S.check_ln_invariants, S.check_sp_sharded_equals_dense,
           S.check_sp_vs_torch, S.check_philox_kat]


def _some_pin_fails(pins):
    for p in pins:
        try:
            if not p():
                return True
        except Exception:  # a shape error is a caught mistake too
            return True
    return False


def _set_gelu(monkeypatch, f=None, fp=None):
    f = f or om.gelu
    fp = fp or om.gelu_prime
    monkeypatch.setattr(om, "gelu", f)
    monkeypatch.setattr(om, "gelu_prime", fp)
    monkeypatch.setitem(om.ACTIVATIONS, "gelu", (f, fp))


def test_dropped_term_in_gelu_prime(monkeypatch):
    _set_gelu(monkeypatch, fp=lambda z: 0.5 * (1.0 + erf(np.asarray(z, float) / np.sqrt(2.0))))
    assert _some_pin_fails(MLP_PINS)


def test_tanh_gelu_instead_of_erf(monkeypatch):
    def tanh_gelu(z):
        z = np.asarray(z, float)
        return 0.5 * z * (1 + np.tanh(np.sqrt(2 / np.pi) * (z + 0.044715 * z ** 3)))
    _set_gelu(monkeypatch, f=tanh_gelu)
    assert _some_pin_fails(MLP_PINS)


def test_wrong_sign_in_gelu(monkeypatch):
    _set_gelu(monkeypatch, f=lambda z: 0.5 * np.asarray(z, float) * (1 - erf(np.asarray(z, float) / np.sqrt(2))))
    assert _some_pin_fails(MLP_PINS)


def test_transposed_weight_gradient(monkeypatch):
    orig = om.shard_backward

    def bad(*a, **k):
        D, dA, dB, dX = orig(*a, **k)
        return D, dA.T if dA.shape[0] == dA.shape[1] else dA[::-1], dB, dX
    monkeypatch.setattr(om, "shard_backward", bad)
    assert _some_pin_fails(MLP_PINS)


def test_input_grad_uses_E_instead_of_D(monkeypatch):
    def bad(X, A_i, B_i, Z, Y, G, act="gelu"):
        E = np.asarray(G, float) @ np.asarray(B_i, float).T
        D = E * om.gelu_prime(Z)
        return D, np.asarray(X, float).T @ D, np.asarray(Y, float).T @ np.asarray(G, float), E @ np.asarray(A_i, float).T
    monkeypatch.setattr(om, "shard_backward", bad)
    assert _some_pin_fails(MLP_PINS)


def test_interleaved_split(monkeypatch):
    monkeypatch.setattr(om, "split_columns", lambda A, t: [np.asarray(A, float)[:, i::t] for i in range(t)])
    assert _some_pin_fails(MLP_PINS)


def test_mean_instead_of_sum(monkeypatch):
    monkeypatch.setattr(om, "reduce_partials",
                        lambda parts: sum(np.asarray(p, float) for p in parts) / len(parts))
    assert _some_pin_fails(MLP_PINS)


def test_unbiased_variance_in_layernorm(monkeypatch):
    def bad(x, gamma, beta, eps):
        x = np.asarray(x, float)
        mean = x.mean(axis=1)
        var = x.var(axis=1, ddof=1)
        rstd = 1 / np.sqrt(var + eps)
        xhat = (x - mean[:, None]) * rstd[:, None]
        return xhat * gamma + beta, mean, rstd, xhat
    monkeypatch.setattr(oln, "ln_forward", bad)
    monkeypatch.setattr(S.oln, "ln_forward", bad)
    import oracle.sp_block as spb
    monkeypatch.setattr(spb, "ln_forward", bad)
    assert _some_pin_fails(SP_PINS)


def test_layernorm_backward_missing_projection(monkeypatch):
    def bad(g, xhat, rstd, gamma):
        gt = np.asarray(g, float) * gamma
        dx = rstd[:, None] * (gt - gt.mean(axis=1, keepdims=True))
        return dx, (g * xhat).sum(axis=0), np.asarray(g).sum(axis=0)
    monkeypatch.setattr(oln, "ln_backward", bad)
    import oracle.sp_block as spb
    monkeypatch.setattr(spb, "ln_backward", bad)
    assert _some_pin_fails(SP_PINS)


def test_philox_swapped_multipliers(monkeypatch):
    monkeypatch.setattr(oph, "M0", 0xCD9E8D57)
    monkeypatch.setattr(oph, "M1", 0xD2511F53)
    assert _some_pin_fails(SP_PINS)


def test_dropout_without_rescale(monkeypatch):
    import oracle.sp_block as spb
    orig_fwd = spb.sp_forward

    def bad_fwd(x, gamma, beta, eps, A, B, t, p, seed):
        f = orig_fwd(x, gamma, beta, eps, A, B, t, p, seed)
        f["out"] = np.asarray(x, float) + f["mask"] * f["mlp"]["O"]
        return f
    monkeypatch.setattr(spb, "sp_forward", bad_fwd)
    monkeypatch.setattr(S.osp, "sp_forward", bad_fwd)
    assert _some_pin_fails(SP_PINS)


@pytest.mark.parametrize("pins", [MLP_PINS, SP_PINS])
def test_unmutated_oracle_passes_every_pin(pins):
    assert not _some_pin_fails(pins)
