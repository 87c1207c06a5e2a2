"""Pins of the fp64 MLP-shard oracle against facts the pages and mathematics fix.

Each check is written so that a plausible mistake in the oracle (a dropped term,
a wrong sign, a transposed operand, a wrong split axis) fails at least one of
them; test_oracle_mutants.py plants such mistakes and checks that they do.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mlp as om
from tpmlp_inputs import config_inputs, mlp_inputs

from conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _c1():
    inp = config_inputs("worked_example", seed=0)
    return inp["X"].f64, inp["A"].f64, inp["B"].f64, inp["G"].f64


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ------------------------------------------------------------------ checks
# Each check returns True when the oracle satisfies the pin.  They are plain
# functions so that the mutant tests can run them against a broken oracle.

def check_gelu_table():
    g = _golden("normal_table.json")
    tol = g["tol"]
    ok = True
    for z, Phi in g["Phi"].items():
        z = float(z)
        ok &= abs(float(om.gelu(z)) - z * Phi) <= tol * max(1.0, abs(z))
    return bool(ok)


def check_gelu_identities():
    z = np.linspace(-6, 6, 241)
    ok = abs(float(om.gelu(0.0))) == 0.0 and abs(float(om.gelu_prime(0.0)) - 0.5) < 1e-15
    ok &= np.max(np.abs(om.gelu(z) - om.gelu(-z) - z)) < 1e-14          # φ(z) − φ(−z) = z
    ok &= np.max(np.abs(om.gelu_prime(z) + om.gelu_prime(-z) - 1.0)) < 1e-14  # φ'(z)+φ'(−z) = 1
    h = 1e-5
    fd = (om.gelu(z + h) - om.gelu(z - h)) / (2 * h)
    ok &= np.max(np.abs(fd - om.gelu_prime(z))) < 1e-9
    return bool(ok)


def check_gelu_vs_torch():
    z = torch.linspace(-8, 8, 1001, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.gelu(z, approximate="none")
    (gz,) = torch.autograd.grad(y.sum(), z)
    zn = z.detach().numpy()
    return bool(np.max(np.abs(om.gelu(zn) - y.detach().numpy())) < 1e-15 * 8
                and np.max(np.abs(om.gelu_prime(zn) - gz.numpy())) < 1e-14)


def check_finite_differences(t=2, step=1e-6):
    """Central differences of ℓ = Σ G⊙O on every entry of X, A and B (the
    worked-example sizes: 12 + 32 + 32 = 76 entries)."""
    X, A, B, G = _c1()
    fwd = om.tp_forward(X, A, B, t)
    bwd = om.tp_backward(X, A, B, fwd, G)
    dA = np.concatenate(bwd["dA"], axis=1)
    dB = np.concatenate(bwd["dB"], axis=0)
    analytic = {"X": bwd["dX"], "A": dA, "B": dB}
    base = {"X": X, "A": A, "B": B}
    worst = 0.0
    for name, arr in base.items():
        for idx in np.ndindex(arr.shape):
            plus = {k: v.copy() for k, v in base.items()}
            minus = {k: v.copy() for k, v in base.items()}
            plus[name][idx] += step
            minus[name][idx] -= step
            lp = om.loss(om.tp_forward(plus["X"], plus["A"], plus["B"], t)["O"], G)
            lm = om.loss(om.tp_forward(minus["X"], minus["A"], minus["B"], t)["O"], G)
            fd = (lp - lm) / (2 * step)
            a = analytic[name][idx]
            worst = max(worst, abs(fd - a) / max(1.0, abs(a)))
    return worst <= 1e-7


def check_torch_autograd(seed=3, n=5, d=8, m=12, t=3):
    """The unsharded layer through torch's own fp64 gelu + autograd."""
    inp = mlp_inputs(n, d, m, t, dtype="f32", seed=seed, x_std=1.0, w_std=0.5, g_std=1.0)
    X, A, B, G = (inp[k].f64 for k in "XABG")
    tx, ta, tb = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    O = torch.nn.functional.gelu(tx @ ta, approximate="none") @ tb
    (O * torch.tensor(G)).sum().backward()
    fwd = om.tp_forward(X, A, B, t)
    bwd = om.tp_backward(X, A, B, fwd, G)
    return bool(relerr(fwd["O"], O.detach().numpy()) < 1e-14
                and relerr(bwd["dX"], tx.grad.numpy()) < 1e-14
                and relerr(np.concatenate(bwd["dA"], 1), ta.grad.numpy()) < 1e-14
                and relerr(np.concatenate(bwd["dB"], 0), tb.grad.numpy()) < 1e-14)


def check_sharded_equals_unsharded(seed=1, n=7, d=16, m=24, ts=(1, 2, 3, 4, 6, 24)):
    """Σ_i φ(XA_i)B_i = φ(XA)B and the matching gradient identities, for every
    divisor t of m including t = 1 (plain MLP) and t = m (one column per shard)."""
    inp = mlp_inputs(n, d, m, 1, dtype="f32", seed=seed, x_std=1.0, w_std=0.3, g_std=1.0)
    X, A, B, G = (inp[k].f64 for k in "XABG")
    O = om.dense_forward(X, A, B)
    dX, dA, dB = om.dense_backward(X, A, B, G)
    ok = True
    for t in ts:
        fwd = om.tp_forward(X, A, B, t)
        bwd = om.tp_backward(X, A, B, fwd, G)
        ok &= relerr(fwd["O"], O) <= 1e-13
        ok &= relerr(bwd["dX"], dX) <= 1e-13
        ok &= relerr(np.concatenate(bwd["dA"], axis=1), dA) <= 1e-13
        ok &= relerr(np.concatenate(bwd["dB"], axis=0), dB) <= 1e-13
        # each local activation block is the matching column block of φ(XA)
        H = om.gelu(X @ A)
        mi = m // t
        for i in range(t):
            ok &= relerr(fwd["Y"][i], H[:, i * mi:(i + 1) * mi]) <= 1e-15
    return bool(ok)


def check_linear_in_G(seed=2):
    """Backward is linear in the upstream gradient ([TRAIN] 前置知识: the
    backward pass is linear, so micro-batch gradients add)."""
    inp = mlp_inputs(6, 8, 16, 2, dtype="f32", seed=seed, x_std=1.0, w_std=0.4, g_std=1.0)
    X, A, B, G1 = (inp[k].f64 for k in "XABG")
    G2 = np.random.default_rng(seed + 100).standard_normal(G1.shape)
    fwd = om.tp_forward(X, A, B, 2)
    b1, b2 = om.tp_backward(X, A, B, fwd, G1), om.tp_backward(X, A, B, fwd, G2)
    b12 = om.tp_backward(X, A, B, fwd, 2.5 * G1 - 0.75 * G2)
    ok = relerr(b12["dX"], 2.5 * b1["dX"] - 0.75 * b2["dX"]) < 1e-13
    for k in ("dA", "dB"):
        for i in range(2):
            ok &= relerr(b12[k][i], 2.5 * b1[k][i] - 0.75 * b2[k][i]) < 1e-13
    return bool(ok)


def check_bruteforce_loops():
    """Pure-Python triple loops (math.erf, no NumPy) for O on the worked
    example: O[r][c] = Σ_j φ(Σ_k X[r][k]·A[k][j])·B[j][c]."""
    X, A, B, _ = _c1()
    n, d = X.shape
    m = A.shape[1]
    O = [[0.0] * d for _ in range(n)]
    for r in range(n):
        for j in range(m):
            h = sum(float(X[r, k]) * float(A[k, j]) for k in range(d))
            y = 0.5 * h * (1.0 + math.erf(h / math.sqrt(2.0)))
            for c in range(d):
                O[r][c] += y * float(B[j, c])
    return relerr(om.tp_forward(X, A, B, 2)["O"], np.array(O)) < 1e-14


# ------------------------------------------------------------------ tests
def test_gelu_matches_normal_table():
    assert check_gelu_table()


def test_gelu_identities_and_derivative():
    assert check_gelu_identities()


def test_gelu_matches_torch_exact_gelu():
    assert check_gelu_vs_torch()


def test_worked_example_shapes():
    g = _golden("worked_example_shapes.json")
    X, A, B, G = _c1()
    assert list(X.shape) == g["X"] and list(A.shape) == g["A"] and list(B.shape) == g["B"]
    fwd = om.tp_forward(X, A, B, g["t"])
    assert len(fwd["Y"]) == g["t"]
    for i in range(g["t"]):
        assert list(om.split_columns(A, 2)[i].shape) == g["A_i"]
        assert list(om.split_rows(B, 2)[i].shape) == g["B_i"]
        assert list(fwd["Y"][i].shape) == g["Y_i"]
        assert list(fwd["P"][i].shape) == g["P_i"]
    assert list(fwd["O"].shape) == g["O"]


def test_worked_example_finite_differences():
    assert check_finite_differences()


def test_worked_example_bruteforce():
    assert check_bruteforce_loops()


def test_matches_torch_autograd():
    assert check_torch_autograd()


def test_sharded_equals_unsharded_all_t():
    assert check_sharded_equals_unsharded()


def test_backward_linear_in_G():
    assert check_linear_in_G()


def test_relu_counterexample():
    g = _golden("relu_counterexample.json")
    X = np.array([[1.0, 1.0]])
    A = np.array([[g["u"]], [g["v"]]])  # X·A = u + v
    B = np.array([[1.0]])
    assert om.dense_forward(X, A, B, act="relu")[0, 0] == g["phi_of_sum"]
    # the method's column split (m = 1, so t = 1) is exact
    assert om.tp_forward(X, A, B, 1, act="relu")["O"][0, 0] == g["phi_of_sum"]
    # the row-first split activates partial sums: φ(u) + φ(v)
    assert om.row_first_split_forward(X, A, B, 2, act="relu")[0, 0] == g["sum_of_phis"]


def test_row_first_split_wrong_with_gelu():
    X, A, B, _ = _c1()
    truth = om.dense_forward(X, A, B)
    assert relerr(om.tp_forward(X, A, B, 2)["O"], truth) < 1e-14
    assert relerr(om.row_first_split_forward(X, A, B, 2), truth) > 1e-2


def test_split_rejects_uneven():
    with pytest.raises(ValueError):
        om.split_columns(np.zeros((4, 10)), 3)
    with pytest.raises(ValueError):
        om.split_rows(np.zeros((10, 4)), 4)
