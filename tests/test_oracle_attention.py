"""Pins of the attention oracle (oracle/attention.py) against things other than
its own formulas: torch's fp64 scaled_dot_product_attention and its autograd
(a library routine for the core, causal or not), central finite differences
through the whole shard, the heads split over shards against the unsplit
layer, the closed form of uniform attention when the queries vanish, and the
shift invariance of the keys (a softmax row is unchanged when all its logits
move together).  The general mask: torch's boolean attn_mask, key padding
against the same attention on the truncated keys, the causal pattern given as
a general mask, rows with every key hidden, and finite differences through a
masked layer.  Plausible mistakes planted in the oracle must fail one of
them."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import attention as oa
from tpmlp_inputs import attn_inputs


def relerr(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _layer(s=5, b=2, d=12, heads=3, seed=0, bias=False):
    inp = attn_inputs(s, b, d, heads, dtype="f32", seed=seed, x_std=1.0, w_std=0.5, g_std=1.0,
                      bias_std=0.5 if bias else None)
    return {k: v.f64 for k, v in inp.items()}


def _qkv(s=6, b=2, nh=3, dh=4, seed=1):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((b, nh, s, dh)) for _ in range(3)]


# ---------------------------------------------------------------- pins
def check_core_vs_torch_sdpa(causal, seed=1):
    """o, and dq, dk, dv for a random upstream do, against torch's fp64
    scaled_dot_product_attention (default scale 1/√dh) and its autograd."""
    q, k, v = _qkv(seed=seed)
    do = np.random.default_rng(seed + 100).standard_normal(q.shape)
    o, A, lse = oa.core_forward(q, k, v, causal)
    dq, dk, dv = oa.core_backward(q, k, v, A, do)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    (to * torch.tensor(do)).sum().backward()
    return bool(relerr(o, to.detach().numpy()) < 1e-13 and relerr(dq, tq.grad.numpy()) < 1e-12
                and relerr(dk, tk.grad.numpy()) < 1e-12 and relerr(dv, tv.grad.numpy()) < 1e-12)


def check_core_causal():
    return check_core_vs_torch_sdpa(True)


def check_core_full():
    return check_core_vs_torch_sdpa(False)


def check_layer_vs_torch(causal=True, t=3, bias=True):
    """The whole layer, heads split over t shards, against torch autograd of
    X·W_qkv + b → (s, b, heads, 3, dh) → SDPA → merge → ·W_proj + b, for every
    gradient including the biases."""
    s, b, d, heads = 5, 2, 12, 3
    L = _layer(s, b, d, heads, seed=4, bias=bias)
    dh = d // heads
    tX, tWq, tWp = (torch.tensor(L[k], requires_grad=True) for k in ("X", "Wqkv", "Wproj"))
    tbq = torch.tensor(L["bqkv"], requires_grad=True) if bias else None
    tbp = torch.tensor(L["bproj"], requires_grad=True) if bias else None
    qkv = tX @ tWq + (tbq if bias else 0)
    T = qkv.reshape(s, b, heads, 3, dh)
    q, k, v = (T[:, :, :, j, :].permute(1, 2, 0, 3) for j in range(3))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=causal)
    Out = o.permute(2, 0, 1, 3).reshape(s * b, d) @ tWp + (tbp if bias else 0)
    (Out * torch.tensor(L["G"])).sum().backward()
    f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, causal,
                      L.get("bqkv") if bias else None, L.get("bproj") if bias else None)
    g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
    ok = relerr(f["Out"], Out.detach().numpy()) < 1e-13
    ok &= relerr(g["dX"], tX.grad.numpy()) < 1e-12
    ok &= relerr(np.concatenate([sh["dWqkv"] for sh in g["shards"]], 1), tWq.grad.numpy()) < 1e-12
    ok &= relerr(np.concatenate([sh["dWproj"] for sh in g["shards"]], 0), tWp.grad.numpy()) < 1e-12
    if bias:
        ok &= relerr(np.concatenate([sh["dbqkv"] for sh in g["shards"]]), tbq.grad.numpy()) < 1e-12
        ok &= relerr(g["dbproj"], tbp.grad.numpy()) < 1e-12
    return bool(ok)


def check_finite_differences(step=1e-6):
    """Central differences of ℓ = Σ G⊙Out on every entry of X, W_qkv, W_proj
    (s = 3, b = 2, d = 4, 2 heads on 2 shards, causal)."""
    s, b, d, heads, t = 3, 2, 4, 2, 2
    L = _layer(s, b, d, heads, seed=7)

    def loss(X, Wq, Wp):
        return float((oa.tp_forward(X, Wq, Wp, t, s, b, heads, True)["Out"] * L["G"]).sum())
    f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, True)
    g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
    grads = {"X": g["dX"], "Wqkv": np.concatenate([sh["dWqkv"] for sh in g["shards"]], 1),
             "Wproj": np.concatenate([sh["dWproj"] for sh in g["shards"]], 0)}
    worst = 0.0
    for name in ("X", "Wqkv", "Wproj"):
        base = L[name]
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                args = {k: L[k].copy() for k in ("X", "Wqkv", "Wproj")}
                args[name][idx] += sgn * step
                vals.append(loss(args["X"], args["Wqkv"], args["Wproj"]))
            fd = (vals[0] - vals[1]) / (2 * step)
            worst = max(worst, abs(fd - grads[name][idx]) / max(1.0, abs(grads[name][idx])))
    return worst <= 1e-7


def check_sharded_equals_unsharded():
    """Splitting the 6 heads over t = 1, 2, 3, 6 shards changes nothing."""
    s, b, d, heads = 4, 3, 24, 6
    L = _layer(s, b, d, heads, seed=2)
    f1 = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], 1, s, b, heads, True)
    g1 = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f1, L["G"])
    ok = True
    for t in (2, 3, 6):
        f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, True)
        g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
        ok &= relerr(f["Out"], f1["Out"]) < 1e-13
        ok &= relerr(g["dX"], g1["dX"]) < 1e-13
        ok &= relerr(np.concatenate([sh["dWqkv"] for sh in g["shards"]], 1), g1["shards"][0]["dWqkv"]) < 1e-13
        ok &= relerr(np.concatenate([sh["dWproj"] for sh in g["shards"]], 0), g1["shards"][0]["dWproj"]) < 1e-13
        ok &= relerr(np.concatenate([sh["O"] for sh in f["shards"]], 1), f1["shards"][0]["O"]) < 1e-13
    return bool(ok)


def check_uniform_attention_closed_form():
    """q = 0: every logit of a row is 0, so attention is uniform over the keys
    it may see: o_i = mean of v_0..v_i (causal) or of all v, lse_i = log(i+1)
    or log(s)."""
    q, k, v = _qkv(s=7, seed=3)
    q = np.zeros_like(q)
    oc, _, lc = oa.core_forward(q, k, v, True)
    of, _, lf = oa.core_forward(q, k, v, False)
    s = q.shape[2]
    prefix = np.cumsum(v, axis=2) / np.arange(1, s + 1)[None, None, :, None]
    ok = relerr(oc, prefix) < 1e-14 and relerr(of, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)) < 1e-14
    ok &= np.allclose(lc, np.log(np.arange(1, s + 1))[None, None, :], rtol=0, atol=1e-14)
    ok &= np.allclose(lf, np.log(s), rtol=0, atol=1e-14)
    return bool(ok)


def check_causal_first_row_and_lse():
    """Causal row 0 sees only key 0: o_0 = v_0; lse is each row's log-sum-exp of
    the scaled, masked logits (scipy)."""
    q, k, v = _qkv(s=5, seed=5)
    o, A, lse = oa.core_forward(q, k, v, True)
    dh = q.shape[3]
    ok = np.allclose(o[:, :, 0, :], v[:, :, 0, :], rtol=0, atol=1e-15)
    for bi in range(q.shape[0]):
        for h in range(q.shape[1]):
            S = q[bi, h] @ k[bi, h].T / np.sqrt(dh)
            S[np.triu_indices(q.shape[2], 1)] = -np.inf
            ok &= np.allclose(lse[bi, h], logsumexp(S, axis=1), rtol=0, atol=1e-13)
    return bool(ok)


def check_key_shift_invariance():
    """Adding one vector u to every key moves each row's logits by q_i·u/√dh,
    which the softmax ignores: o is unchanged, and so Σ_j dk_j = 0 for every
    (batch entry, head)."""
    q, k, v = _qkv(s=6, seed=8)
    do = np.random.default_rng(9).standard_normal(q.shape)
    u = np.random.default_rng(10).standard_normal(q.shape[3])
    o0, A, _ = oa.core_forward(q, k, v, True)
    o1, _, _ = oa.core_forward(q, k + u, v, True)
    _, dk, _ = oa.core_backward(q, k, v, A, do)
    return bool(relerr(o1, o0) < 1e-13 and np.abs(dk.sum(axis=2)).max() < 1e-12)


def _mask(b, s, seed, p=0.4, keep_diag=True):
    """Random boolean mask [b, s, s] (True hides the key); with keep_diag every
    query sees at least its own position."""
    m = np.random.default_rng(seed).random((b, s, s)) < p
    if keep_diag:
        m[:, np.arange(s), np.arange(s)] = False
    return m


def check_mask_vs_torch_sdpa():
    """A random general mask, alone and with the causal one, against torch's
    fp64 SDPA with the boolean attn_mask (True there = may attend) and its
    autograd; every row keeps at least one key."""
    q, k, v = _qkv(s=7, seed=11)
    b, nh, s, dh = q.shape
    do = np.random.default_rng(12).standard_normal(q.shape)
    m = _mask(b, s, 13)
    ok = True
    for causal in (False, True):
        o, A, lse = oa.core_forward(q, k, v, causal, m)
        dq, dk, dv = oa.core_backward(q, k, v, A, do)
        allow = ~m & (np.tril(np.ones((s, s), bool)) if causal else True)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(allow)[:, None])
        (to * torch.tensor(do)).sum().backward()
        ok &= relerr(o, to.detach().numpy()) < 1e-13 and relerr(dq, tq.grad.numpy()) < 1e-12
        ok &= relerr(dk, tk.grad.numpy()) < 1e-12 and relerr(dv, tv.grad.numpy()) < 1e-12
    return bool(ok)


def check_key_padding_is_truncation():
    """Hiding keys j >= L_β (a padding mask) equals attention over the first
    L_β keys only; the hidden keys get zero dk, dv."""
    q, k, v = _qkv(s=8, b=3, seed=14)
    b, nh, s, dh = q.shape
    do = np.random.default_rng(15).standard_normal(q.shape)
    L = [8, 5, 3]
    m = np.zeros((b, s, s), bool)
    for bi, n in enumerate(L):
        m[bi, :, n:] = True
    ok = True
    for causal in (False, True):
        o, A, lse = oa.core_forward(q, k, v, causal, m)
        dq, dk, dv = oa.core_backward(q, k, v, A, do)
        for bi, n in enumerate(L):
            sl = (slice(bi, bi + 1), slice(None))
            q1, k1, v1 = q[sl], k[sl][:, :, :n], v[sl][:, :, :n]
            # truncated keys, all queries: the causal pattern of a query i >= n
            # sees every kept key, which tril on an [s, n] block expresses
            keep = np.tril(np.ones((s, n), bool)) if causal else np.ones((s, n), bool)
            S = np.einsum("bhid,bhjd->bhij", q1, k1) / np.sqrt(dh)
            S = np.where(keep, S, -np.inf)
            At = np.exp(S - S.max(-1, keepdims=True))
            At /= At.sum(-1, keepdims=True)
            ok &= relerr(o[sl], At @ v1) < 1e-13
            ok &= np.allclose(lse[sl], logsumexp(S, axis=-1), rtol=0, atol=1e-13)
            ok &= np.all(dk[sl][:, :, n:] == 0) and np.all(dv[sl][:, :, n:] == 0)
            dP = do[sl] @ np.swapaxes(v1, -1, -2)
            dS = At * (dP - (dP * At).sum(-1, keepdims=True))
            ok &= relerr(dq[sl], dS @ k1 / np.sqrt(dh)) < 1e-12
            ok &= relerr(dk[sl][:, :, :n], np.swapaxes(dS, -1, -2) @ q1 / np.sqrt(dh)) < 1e-12
    return bool(ok)


def check_causal_pattern_as_general_mask():
    q, k, v = _qkv(s=6, seed=16)
    b, s = q.shape[0], q.shape[2]
    m = np.broadcast_to(np.triu(np.ones((s, s), bool), 1), (b, s, s))
    o1, A1, l1 = oa.core_forward(q, k, v, True)
    o2, A2, l2 = oa.core_forward(q, k, v, False, m)
    return bool(np.array_equal(o1, o2) and np.array_equal(A1, A2) and np.array_equal(l1, l2))


def check_rows_with_every_key_hidden():
    """A query that may see no key: o = 0, lse = −∞, dq = 0; the other rows are
    those of the same mask with that row opened to a single key."""
    q, k, v = _qkv(s=6, seed=17)
    b, nh, s, dh = q.shape
    do = np.random.default_rng(18).standard_normal(q.shape)
    m = _mask(b, s, 19)
    m[0, 2, :] = True
    m[1, 0, :] = True
    o, A, lse = oa.core_forward(q, k, v, False, m)
    dq, dk, dv = oa.core_backward(q, k, v, A, do)
    ok = np.all(o[0, :, 2] == 0) and np.all(o[1, :, 0] == 0)
    ok &= np.all(np.isneginf(lse[0, :, 2])) and np.all(np.isneginf(lse[1, :, 0]))
    ok &= np.all(dq[0, :, 2] == 0) and np.all(dq[1, :, 0] == 0) and np.all(np.isfinite(dk))
    m2 = m.copy()
    m2[0, 2, 0] = False
    m2[1, 0, 0] = False
    o2, _, _ = oa.core_forward(q, k, v, False, m2)
    rows = np.ones((b, s), bool)
    rows[0, 2] = rows[1, 0] = False
    ok &= np.array_equal(o.transpose(0, 2, 1, 3)[rows], o2.transpose(0, 2, 1, 3)[rows])
    return bool(ok)


def check_masked_finite_differences(step=1e-6):
    """Central differences of ℓ = Σ G⊙Out on every entry of X, W_qkv, W_proj
    through a layer with a general mask (one query row fully hidden), causal."""
    s, b, d, heads, t = 4, 2, 4, 2, 2
    L = _layer(s, b, d, heads, seed=21)
    m = _mask(b, s, 22, p=0.5, keep_diag=False)
    m[1, 3, :] = True

    def fwd(X, Wq, Wp):
        return oa.tp_forward(X, Wq, Wp, t, s, b, heads, True, mask=m)
    f = fwd(L["X"], L["Wqkv"], L["Wproj"])
    g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
    grads = {"X": g["dX"], "Wqkv": np.concatenate([sh["dWqkv"] for sh in g["shards"]], 1),
             "Wproj": np.concatenate([sh["dWproj"] for sh in g["shards"]], 0)}
    worst = 0.0
    for name in ("X", "Wqkv", "Wproj"):
        for idx in np.ndindex(L[name].shape):
            vals = []
            for sgn in (1.0, -1.0):
                args = {kk: L[kk].copy() for kk in ("X", "Wqkv", "Wproj")}
                args[name][idx] += sgn * step
                vals.append(float((fwd(args["X"], args["Wqkv"], args["Wproj"])["Out"] * L["G"]).sum()))
            fd = (vals[0] - vals[1]) / (2 * step)
            worst = max(worst, abs(fd - grads[name][idx]) / max(1.0, abs(grads[name][idx])))
    return worst <= 1e-7


PINS = [check_core_causal, check_core_full, check_layer_vs_torch, check_finite_differences,
        check_sharded_equals_unsharded, check_uniform_attention_closed_form,
        check_causal_first_row_and_lse, check_key_shift_invariance, check_mask_vs_torch_sdpa,
        check_key_padding_is_truncation, check_causal_pattern_as_general_mask,
        check_rows_with_every_key_hidden, check_masked_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    assert pin()


def _some_pin_fails():
    for p in PINS:
        try:
            if not p():
                return True
        except Exception:
            return True
    return False


def _mutant_core(monkeypatch, transform_S=None, transform_keep=None, dS_rule=None, dk_rule=None,
                 transform_mask=None):
    """Re-plant core_forward / core_backward with one step changed."""
    def fwd(q, k, v, causal, mask=None):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        b, nh, s, dh = q.shape
        o, A, lse = np.zeros_like(q), np.zeros((b, nh, s, s)), np.zeros((b, nh, s))
        base = np.tril(np.ones((s, s), bool)) if causal else np.ones((s, s), bool)
        if transform_keep:
            base = transform_keep(base, causal)
        for bi in range(b):
            keep = base
            if mask is not None:
                mb = np.asarray(mask[bi], bool)
                keep = base & ~(transform_mask(mb) if transform_mask else mb)
            seen = keep.any(axis=1)
            for h in range(nh):
                S = q[bi, h] @ k[bi, h].T / np.sqrt(dh)
                if transform_S:
                    S = transform_S(S, dh)
                S = np.where(keep, S, -np.inf)
                mx = np.where(seen, S.max(axis=1), 0.0)[:, None]
                E = np.exp(S - mx)
                z = np.where(seen[:, None], E.sum(axis=1, keepdims=True), 1.0)
                A[bi, h] = E / z
                lse[bi, h] = np.where(seen, mx[:, 0] + np.log(z[:, 0]), -np.inf)
                o[bi, h] = A[bi, h] @ v[bi, h]
        return o, A, lse

    def bwd(q, k, v, A, do):
        q, k, v, A, do = (np.asarray(x, np.float64) for x in (q, k, v, A, do))
        b, nh, s, dh = q.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for bi in range(b):
            for h in range(nh):
                P = A[bi, h]
                dv[bi, h] = P.T @ do[bi, h]
                dP = do[bi, h] @ v[bi, h].T
                dS = dS_rule(P, dP) if dS_rule else P * (dP - (dP * P).sum(axis=1, keepdims=True))
                dq[bi, h] = dS @ k[bi, h] / np.sqrt(dh)
                dk[bi, h] = (dk_rule(dS, q[bi, h]) if dk_rule else dS.T @ q[bi, h]) / np.sqrt(dh)
        return dq, dk, dv
    monkeypatch.setattr(oa, "core_forward", fwd)
    monkeypatch.setattr(oa, "core_backward", bwd)


def test_mutant_missing_scale(monkeypatch):
    _mutant_core(monkeypatch, transform_S=lambda S, dh: S * np.sqrt(dh))
    assert _some_pin_fails()


def test_mutant_causal_mask_off_by_one(monkeypatch):
    """Each query also sees the next token."""
    _mutant_core(monkeypatch, transform_keep=lambda keep, causal: np.tril(np.ones_like(keep), 1) if causal else keep)
    assert _some_pin_fails()


def test_mutant_causal_mask_transposed(monkeypatch):
    _mutant_core(monkeypatch, transform_keep=lambda keep, causal: keep.T)
    assert _some_pin_fails()


def test_mutant_softmax_gradient_without_rowsum(monkeypatch):
    _mutant_core(monkeypatch, dS_rule=lambda P, dP: P * dP)
    assert _some_pin_fails()


def test_mutant_dk_without_transpose(monkeypatch):
    _mutant_core(monkeypatch, dk_rule=lambda dS, q: dS @ q)
    assert _some_pin_fails()


def test_mutant_head_column_order(monkeypatch):
    """Reading W_qkv's columns as (q|k|v, head, dh) instead of (head, q|k|v, dh)."""
    def split(QKV, s, b, nh, dh):
        T = np.asarray(QKV, np.float64).reshape(s, b, 3, nh, dh)
        return tuple(T[:, :, j].transpose(1, 2, 0, 3) for j in range(3))

    def merge(dq, dk, dv):
        b, nh, s, dh = dq.shape
        return np.stack([dq, dk, dv], axis=2).transpose(3, 0, 2, 1, 4).reshape(s * b, 3 * nh * dh)
    monkeypatch.setattr(oa, "split_heads", split)
    monkeypatch.setattr(oa, "merge_qkv", merge)
    assert _some_pin_fails()


def test_mutant_general_mask_transposed(monkeypatch):
    """mask[β][j][i] read for query i, key j."""
    _mutant_core(monkeypatch, transform_mask=lambda mb: mb.T)
    assert _some_pin_fails()


def test_mutant_general_mask_ignored(monkeypatch):
    _mutant_core(monkeypatch, transform_mask=lambda mb: np.zeros_like(mb))
    assert _some_pin_fails()


def test_mutant_general_mask_off_by_one(monkeypatch):
    """The mask read one key to the right (key j uses the bit of key j + 1)."""
    _mutant_core(monkeypatch, transform_mask=lambda mb: np.concatenate([mb[:, 1:], mb[:, :1]], axis=1))
    assert _some_pin_fails()
