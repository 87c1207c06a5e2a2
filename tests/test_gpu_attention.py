"""GPU parity of the self-attention shard (tpmlp_attn_core_fwd/_bwd and
tpmlp_attn_fwd/_bwd) against the fp64 oracle (oracle/attention.py) on the
same seeded inputs, through the C ABI.

Bars (relative Frobenius error, fp64): fp32 path 1e-5, bf16 path 8e-3, for
every output and gradient (o, lse, dq, dk, dv; QKV, O, P, the summed output,
dO, dQKV, dW_qkv, dW_proj, dX).  lse is compared as exp(lse) (the row's
softmax normaliser), whose relative error is lse's absolute error.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from oracle import attention as oa
from tpmlp_inputs import CONFIGS, Tensor, attn_inputs, attn_mask, config_inputs, f32_to_bf16_bits, qkv_inputs

from gpu_util import dev, f64, relerr, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 8e-3}


def lse_err(gpu, ref):
    """Relative Frobenius error of the softmax normalisers exp(lse)."""
    return relerr(np.exp(f64(gpu)), np.exp(np.asarray(ref, np.float64)))


# ------------------------------------------------------------------ the core
def run_core(inp, T, s, b, nh, dh, causal, mask=None):
    qkv, do = dev(inp["qkv"]), dev(inp["do"])
    m = None if mask is None else torch.from_numpy(mask).cuda()
    o = torch.empty((T, s * b, nh * dh), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((T, b, nh, s), dtype=torch.float32, device="cuda")
    tp.tpmlp_attn_core_fwd(qkv, o, lse, s, b, nh, dh, causal, mask=m)
    dqkv = torch.empty_like(qkv)
    ws = torch.empty(max(tp.attn_bwd_workspace_bytes(T, s, b, nh), 4), dtype=torch.uint8, device="cuda")
    tp.tpmlp_attn_core_bwd(qkv, o, lse, do, dqkv, ws, s, b, nh, dh, causal, mask=m)
    torch.cuda.synchronize()
    return o, lse, dqkv


def compare_core(T, s, b, nh, dh, causal, dtype, seed=0, inp=None, mask=None):
    say(f"[gpu] attention core {dtype} T={T} s={s} b={b} nh={nh} dh={dh} causal={causal} "
        f"mask={'none' if mask is None else 'general'}")
    if inp is None:
        inp = qkv_inputs(T, s, b, nh, dh, dtype=dtype, seed=seed)
    o, lse, dqkv = run_core(inp, T, s, b, nh, dh, causal, mask)
    tol = TOL[dtype]
    errs = {}
    for i in range(T):
        q, k, v = oa.split_heads(inp["qkv"].f64[i], s, b, nh, dh)
        do = oa.unmerge_heads(inp["do"].f64[i], s, b, nh, dh)
        ro, A, rlse = oa.core_forward(q, k, v, causal, None if mask is None else mask.astype(bool))
        dq, dk, dv = oa.core_backward(q, k, v, A, do)
        errs[f"o{i}"] = relerr(o[i], oa.merge_heads(ro))
        errs[f"dqkv{i}"] = relerr(dqkv[i], oa.merge_qkv(dq, dk, dv))
        gq, gk, gv = oa.split_heads(f64(dqkv[i]), s, b, nh, dh)
        errs[f"dq{i}"], errs[f"dk{i}"], errs[f"dv{i}"] = relerr(gq, dq), relerr(gk, dk), relerr(gv, dv)
        errs[f"lse{i}"] = lse_err(lse[i], rlse)
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] attention core: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"


@pytest.mark.parametrize("T,s,b,nh,dh,causal", [
    (1, 1, 1, 1, 64, True),
    (1, 5, 2, 2, 64, False),
    (2, 70, 2, 1, 64, True),
    (1, 33, 1, 2, 128, True),
    (1, 130, 3, 1, 128, False),
])
def test_core_fp32(T, s, b, nh, dh, causal):
    compare_core(T, s, b, nh, dh, causal, "f32")


@pytest.mark.parametrize("T,s,b,nh,dh,causal", [
    (1, 1, 1, 1, 64, True),      # one token: o = v
    (1, 5, 2, 2, 64, False),     # one partial key tile
    (2, 63, 1, 2, 64, True),
    (1, 64, 2, 1, 128, True),    # exactly one key tile
    (1, 65, 1, 1, 128, True),    # one row into the second tile
    (2, 130, 3, 3, 128, False),  # two query blocks, ragged
    (1, 300, 2, 2, 128, True),   # several query blocks and key tiles
    (1, 257, 1, 2, 64, True),
])
def test_core_bf16(T, s, b, nh, dh, causal):
    compare_core(T, s, b, nh, dh, causal, "bf16")


@pytest.mark.parametrize("T,s,b,nh,dh", [
    (1, 320, 2, 2, 128),
    (1, 384, 1, 3, 128),   # six key tiles, three workgroups of keys, three heads
    (2, 200, 2, 1, 128),   # ragged: the last key tile holds 8 keys
    (1, 384, 2, 2, 64),
])
@pytest.mark.parametrize("causal", [True, False])
def test_core_bf16_growing_logits(causal, T, s, b, nh, dh):
    """Keys scaled by 2^⌊j/64⌋ (exact in bf16): every key tile doubles the
    logits' spread, so the row maxima grow by less than the forward's rescale
    threshold on the early tiles (P well above 1 against a stale reference)
    and by more on the later ones (the reference moves mid-row); the
    backward's P and dS are then concentrated on few keys per row."""
    inp = qkv_inputs(T, s, b, nh, dh, dtype="bf16", seed=8)
    x = inp["qkv"].f32.reshape(T, s, b, nh, 3, dh).copy()
    x[:, :, :, :, 1, :] *= (2.0 ** (np.arange(s) // 64)).astype(np.float32)[None, :, None, None, None]
    inp["qkv"] = Tensor(f32_to_bf16_bits(x.reshape(T, s * b, nh * 3 * dh)), "bf16")
    assert np.array_equal(inp["qkv"].f32.reshape(x.shape), x)  # the scaling is exact
    compare_core(T, s, b, nh, dh, causal, "bf16", inp=inp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,s,b,nh,dh,causal,kind", [
    (1, 5, 2, 2, 64, False, "random"),
    (1, 70, 2, 1, 64, True, "padding"),     # padded query rows see no key
    (2, 130, 3, 1, 128, False, "padding"),
    (1, 130, 2, 2, 128, True, "random"),
    (1, 257, 2, 1, 128, False, "random"),   # s % 4 != 0: byte-wise mask reads
    (1, 256, 2, 2, 64, False, "random"),    # s % 4 == 0: word-wise mask reads
])
def test_core_general_mask(T, s, b, nh, dh, causal, kind, dtype):
    """The general mask (BERT-style padding, or random entries), alone or with
    the causal one, against the oracle's masked core; rows that see no key
    must come out as o = 0, lse = −∞, no gradient."""
    mask = attn_mask(b, s, kind, seed=s)
    compare_core(T, s, b, nh, dh, causal, dtype, seed=1, mask=mask)


@pytest.mark.parametrize("b,s", [(1, 1), (2, 33), (3, 64), (2, 100)])
def test_pack_mask_bits(b, s):
    """The packed mask against NumPy's bit packing of the same bytes: part 0
    by query row, part 1 by key column (the transpose), positions past s set."""
    m = attn_mask(b, s, "random", seed=b * 100 + s, p=0.4)
    packed = tp.attn_pack_mask(torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    W = (s + 31) // 32
    pad = np.ones((b, s, 32 * W), np.uint8)
    rows, cols = pad.copy(), pad.copy()
    rows[:, :, :s] = m != 0
    cols[:, :, :s] = np.swapaxes(m, 1, 2) != 0
    ref = np.stack([np.packbits(x, axis=-1, bitorder="little").view(np.uint32).reshape(b, s, W)
                    for x in (rows, cols)])
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), ref)


def test_core_rows_with_no_visible_key():
    """Rows whose every key is hidden: exactly zero output and dq, lse = −∞."""
    T, s, b, nh, dh = 1, 100, 2, 2, 128
    mask = attn_mask(b, s, "random", seed=5, p=0.2)
    mask[0, 7, :] = 1
    mask[1, 64:70, :] = 1
    inp = qkv_inputs(T, s, b, nh, dh, dtype="bf16", seed=2)
    o, lse, dqkv = run_core(inp, T, s, b, nh, dh, False, mask)
    o4 = f64(o).reshape(s, b, nh, dh)
    dq4 = f64(dqkv).reshape(s, b, nh, 3, dh)[:, :, :, 0, :]
    l4 = f64(lse)[0]
    for bi, rows in ((0, [7]), (1, list(range(64, 70)))):
        assert np.all(o4[rows, bi] == 0) and np.all(dq4[rows, bi] == 0)
        assert np.all(np.isneginf(l4[bi][:, rows]))
    assert np.all(np.isfinite(f64(dqkv)))


@pytest.mark.parametrize("T,s,b,nh", [
    (1, 256, 16, 16),   # 512 key blocks of 128 on 256 CUs: the persistent dk/dv kernel, two per workgroup
    (2, 200, 8, 16),    # two shards, ragged: each sequence's last key block holds 72 keys
    (1, 384, 16, 11),   # 528 blocks: some workgroups walk three
])
@pytest.mark.parametrize("causal", [True, False])
def test_core_bf16_persistent_dkdv(T, s, b, nh, causal):
    """dh 128 launches with at least 512 key blocks (a multiple of the 8 XCDs)
    run dk/dv persistently: each workgroup walks several key blocks and loads
    the next block's rows while the current one runs."""
    compare_core(T, s, b, nh, 128, causal, "bf16", seed=11)


def test_core_persistent_dkdv_deterministic_bitwise():
    inp = qkv_inputs(1, 384, 16, 11, 128, dtype="bf16", seed=12)
    r1 = run_core(inp, 1, 384, 16, 11, 128, True)
    r2 = run_core(inp, 1, 384, 16, 11, 128, True)
    for x, y in zip(r1, r2):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_core_deterministic_bitwise():
    inp = qkv_inputs(2, 200, 2, 2, 128, dtype="bf16", seed=4)
    r1 = run_core(inp, 2, 200, 2, 2, 128, True)
    r2 = run_core(inp, 2, 200, 2, 2, 128, True)
    for x, y in zip(r1, r2):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_core_uniform_when_queries_vanish():
    """q = 0: the causal output row i is the mean of v_0..v_i (closed form)."""
    T, s, b, nh, dh = 1, 150, 2, 1, 64
    inp = qkv_inputs(T, s, b, nh, dh, dtype="bf16", seed=6)
    qkv = dev(inp["qkv"])
    qkv.view(T, s, b, nh, 3, dh)[:, :, :, :, 0, :] = 0
    o = torch.empty((T, s * b, nh * dh), dtype=qkv.dtype, device="cuda")
    lse = torch.empty((T, b, nh, s), dtype=torch.float32, device="cuda")
    tp.tpmlp_attn_core_fwd(qkv, o, lse, s, b, nh, dh, True)
    torch.cuda.synchronize()
    v = f64(qkv).reshape(T, s, b, nh, 3, dh)[0, :, :, 0, 2, :]       # [s, b, dh]
    ref = np.cumsum(v, axis=0) / np.arange(1, s + 1)[:, None, None]
    assert relerr(f64(o).reshape(s, b, dh), ref) <= TOL["bf16"]
    assert np.allclose(f64(lse)[0, :, 0, :], np.log(np.arange(1, s + 1))[None, :], rtol=0, atol=1e-5)


# ------------------------------------------------------------------ the layer
def run_layer(inp, s, b, heads, t, causal, mask=None):
    X, Wq, Wp, G = (dev(inp[k]) for k in ("X", "Wqkv", "Wproj", "G"))
    dh = X.shape[1] // heads
    m = None if mask is None else torch.from_numpy(mask).cuda()
    Wq_s, Wp_s = shard_cols(Wq, t), shard_rows(Wp, t)
    QKV, O, lse, P = tp.attn_fwd(X, Wq_s, Wp_s, s, b, dh, causal, mask=m)
    Out = tp.reduce_partials(P)
    dO, dQKV, dWqkv, dWproj, dXp = tp.attn_bwd(X, Wq_s, Wp_s, QKV, O, lse, G, s, b, dh, causal, mask=m)
    dX = tp.reduce_partials(dXp)
    torch.cuda.synchronize()
    return dict(QKV=QKV, O=O, lse=lse, P=P, Out=Out, dO=dO, dQKV=dQKV, dWqkv=dWqkv, dWproj=dWproj, dXp=dXp, dX=dX)


def compare_layer(s, b, d, heads, t, causal, dtype, seed=0, mask=None):
    # weights of std 1.2/√d give logits of std ≈ 1.4 (w²·d), as the 0.02
    # initialisation does at d = 3072; larger ones make the softmax one-hot
    # and the fp32 logits' rounding dominate the comparison
    say(f"[gpu] attention layer {dtype} s={s} b={b} d={d} heads={heads} t={t} causal={causal}")
    inp = attn_inputs(s, b, d, heads, dtype=dtype, seed=seed, x_std=1.0, w_std=1.2 / np.sqrt(d), g_std=1.0)
    r = run_layer(inp, s, b, heads, t, causal, mask)
    L = {k: v.f64 for k, v in inp.items()}
    f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, causal,
                      mask=None if mask is None else mask.astype(bool))
    g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
    tol = TOL[dtype]
    errs = {"Out": relerr(r["Out"], f["Out"]), "dX": relerr(r["dX"], g["dX"])}
    for i in range(t):
        fs, gs = f["shards"][i], g["shards"][i]
        for k, ref in (("QKV", fs["QKV"]), ("O", fs["O"]), ("P", fs["P"]), ("dO", gs["dO"]),
                       ("dQKV", gs["dQKV"]), ("dWqkv", gs["dWqkv"]), ("dWproj", gs["dWproj"]),
                       ("dXp", gs["dXp"])):
            errs[f"{k}{i}"] = relerr(r[k][i], ref)
        errs[f"lse{i}"] = lse_err(r["lse"][i], fs["lse"])
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] attention layer: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"


@pytest.mark.parametrize("s,b,d,heads,t,causal", [
    (5, 2, 128, 2, 2, True),
    (40, 1, 256, 2, 1, False),
])
def test_layer_fp32(s, b, d, heads, t, causal):
    compare_layer(s, b, d, heads, t, causal, "f32")


@pytest.mark.parametrize("s,b,d,heads,t,causal", [
    (5, 2, 128, 2, 2, True),
    (70, 3, 256, 4, 2, True),      # dh = 64
    (130, 2, 512, 4, 2, False),    # dh = 128
    (200, 2, 768, 6, 3, True),
])
def test_layer_bf16(s, b, d, heads, t, causal):
    compare_layer(s, b, d, heads, t, causal, "bf16")


def test_gpt8p3b_attention_shard0_full():
    """h = 3072, 24 heads of 128, t = 8 (3 heads per shard), b = 8, s = 1024,
    causal: all 8 shards on the GPU; shard 0 compared in full with the oracle
    computing that shard from scratch (its QKV, attention, projection and
    every gradient), plus sampled rows of the summed output's input
    gradient partial of shard 7."""
    c = CONFIGS["gpt8p3b_attn_t8"]
    s, b, d, heads, t, causal = c["s"], c["b"], c["d"], c["heads"], c["t"], c["causal"]
    inp = config_inputs("gpt8p3b_attn_t8", seed=0)
    say(f"[gpu] 8.3B-shaped attention: s={s} b={b} d={d} heads={heads} t={t}")
    r = run_layer(inp, s, b, heads, t, causal)
    nh = heads // t
    Xf, Gf = inp["X"].f32, inp["G"].f32
    Wq, Wp = inp["Wqkv"].f32, inp["Wproj"].f32
    w = d // t
    errs = {}
    for i in (0, 7):
        Wq_i, Wp_i = Wq[:, 3 * w * i:3 * w * (i + 1)], Wp[w * i:w * (i + 1), :]
        fs = oa.shard_forward(Xf, Wq_i, Wp_i, s, b, nh, causal)
        gs = oa.shard_backward(Xf, Wq_i, Wp_i, fs, Gf, s, b, nh)
        for k, ref in (("QKV", fs["QKV"]), ("O", fs["O"]), ("P", fs["P"]), ("dO", gs["dO"]),
                       ("dQKV", gs["dQKV"]), ("dWqkv", gs["dWqkv"]), ("dWproj", gs["dWproj"]),
                       ("dXp", gs["dXp"])):
            errs[f"{k}{i}"] = relerr(r[k][i], ref)
        errs[f"lse{i}"] = lse_err(r["lse"][i], fs["lse"])
        del fs, gs
    bad = {k: e for k, e in errs.items() if not (e <= TOL["bf16"])}
    say(f"[gpu] 8.3B-shaped attention: worst {max(errs.values()):.3e}")
    assert not bad, f"over {TOL['bf16']}: {bad}"
    del r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_padding_mask(dtype):
    """The layer with a BERT-style padding mask (non-causal), heads over 2 shards."""
    s, b = 90, 3
    compare_layer(s, b, 256, 4, 2, False, dtype, seed=3, mask=attn_mask(b, s, "padding", seed=9))


@pytest.mark.parametrize("dtype,causal", [("f32", True), ("bf16", True), ("bf16", False)])
def test_layer_with_biases(dtype, causal):
    """QKV bias in the QKV GEMM's epilogue (tpmlp_attn_fwd_bias), the
    projection bias after the sum (tpmlp_reduce_partials_bias), and both bias
    gradients as column sums (tpmlp_bias_grad), against the oracle's biased
    layer."""
    s, b, d, heads, t = 70, 2, 256, 4, 2
    say(f"[gpu] attention layer with biases {dtype} causal={causal}")
    inp = attn_inputs(s, b, d, heads, dtype=dtype, seed=4, x_std=1.0, w_std=1.2 / np.sqrt(d), g_std=1.0,
                      bias_std=0.5)
    X, Wq, Wp, G = (dev(inp[k]) for k in ("X", "Wqkv", "Wproj", "G"))
    bq, bp = dev(inp["bqkv"]), dev(inp["bproj"])
    dh = d // heads
    Wq_s, Wp_s = shard_cols(Wq, t), shard_rows(Wp, t)
    bq_s = bq.reshape(t, 3 * d // t).contiguous()
    QKV, O, lse, P = tp.attn_fwd(X, Wq_s, Wp_s, s, b, dh, causal, bqkv=bq_s)
    Out = tp.reduce_partials_bias(P, bp)
    dO, dQKV, dWqkv, dWproj, dXp = tp.attn_bwd(X, Wq_s, Wp_s, QKV, O, lse, G, s, b, dh, causal)
    dX = tp.reduce_partials(dXp)
    dbq = tp.bias_grad(dQKV)
    dbp = tp.bias_grad(G)
    torch.cuda.synchronize()
    L = {k: v.f64 for k, v in inp.items()}
    f = oa.tp_forward(L["X"], L["Wqkv"], L["Wproj"], t, s, b, heads, causal, bqkv=L["bqkv"], bproj=L["bproj"])
    g = oa.tp_backward(L["X"], L["Wqkv"], L["Wproj"], f, L["G"])
    errs = {"Out": relerr(Out, f["Out"]), "dX": relerr(dX, g["dX"]), "dbproj": relerr(dbp, g["dbproj"])}
    for i in range(t):
        errs[f"QKV{i}"] = relerr(QKV[i], f["shards"][i]["QKV"])
        errs[f"dQKV{i}"] = relerr(dQKV[i], g["shards"][i]["dQKV"])
        errs[f"dbqkv{i}"] = relerr(dbq[i], g["shards"][i]["dbqkv"])
        errs[f"dWqkv{i}"] = relerr(dWqkv[i], g["shards"][i]["dWqkv"])
    tol = TOL[dtype]
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    say(f"[gpu] attention layer with biases: worst {max(errs.values()):.3e}")
    assert not bad, f"over {tol}: {bad}"
