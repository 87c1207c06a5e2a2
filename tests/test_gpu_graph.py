"""Whole steps captured into a HIP graph and replayed: the MLP shard step (tpmlp_fwd,
tpmlp_reduce_partials, tpmlp_bwd, tpmlp_reduce_partials), the attention side of the
layer (causal, or with a packed padding mask) and the vocabulary-parallel cross-entropy.

The library only enqueues kernels on the caller's stream: it allocates, clears and
synchronises nothing, so the whole step can be captured once and replayed.  Every replay
reads the inputs as they are at replay time; the kernels are deterministic, so each replay
must reproduce the eager step bit for bit.  Eager work and synchronisations run between
the replays, and the inputs change between them, so a replay that reused stale results or
skipped a node would show.
"""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
from tpmlp_inputs import attn_inputs, attn_mask, mlp_inputs, vocab_inputs

from gpu_util import dev, say, shard_cols, shard_rows

pytestmark = pytest.mark.gpu

OUTS = ("Z", "Y", "P", "O", "D", "dA", "dB", "dXp", "dX")


def _buffers(X, A, B):
    t, d, mi = A.shape
    n = X.shape[0]
    e = dict(device=X.device)
    return dict(
        Z=torch.empty((t, n, mi), dtype=X.dtype, **e),
        Y=torch.empty((t, n, mi), dtype=X.dtype, **e),
        P=torch.empty((t, n, d), dtype=X.dtype, **e),
        O=torch.empty((n, d), dtype=X.dtype, **e),
        D=torch.empty((t, n, mi), dtype=X.dtype, **e),
        dA=torch.empty((t, d, mi), dtype=torch.float32, **e),
        dB=torch.empty((t, mi, d), dtype=torch.float32, **e),
        dXp=torch.empty((t, n, d), dtype=X.dtype, **e),
        dX=torch.empty((n, d), dtype=X.dtype, **e),
        ws=torch.empty(max(tp.bwd_workspace_bytes(X, A), 16), dtype=torch.uint8, **e),
        wsf=torch.empty(max(tp.fwd_workspace_bytes(X, A), 16), dtype=torch.uint8, **e),
    )


def _step(X, A, B, G, o):
    tp.tpmlp_fwd(X, A, B, o["Z"], o["Y"], o["P"], o["wsf"])
    tp.tpmlp_reduce_partials(o["P"], o["O"])
    tp.tpmlp_bwd(X, A, B, o["Z"], o["Y"], G, o["D"], o["dA"], o["dB"], o["dXp"], o["ws"])
    tp.tpmlp_reduce_partials(o["dXp"], o["dX"])


@pytest.mark.parametrize("dtype,n,d,m,t,policy", [
    ("bf16", 520, 264, 512, 4, tp.GEMM_TILE_AUTO), ("f32", 130, 72, 96, 3, tp.GEMM_TILE_AUTO),
    # K-split products (the fix-up kernels are captured too)
    ("bf16", 256, 2048, 512, 1, tp.GEMM_TILE_AUTO),
    # the single-shard layer: 256x128 tiles for GEMM1 and dgrad-1, K-split P = Y·B
    ("bf16", 2048, 1024, 4096, 1, tp.GEMM_TILE_AUTO),
    # a K-split tail (16 tail tiles in 4 pieces) for GEMM1 and dgrad-1
    ("bf16", 4352, 256, 4096, 1, tp.GEMM_STREAMK),
])
def test_step_graph_replays_match_eager(dtype, n, d, m, t, policy):
    say(f"[gpu] graph capture {dtype} n={n} d={d} m={m} t={t} policy={policy}")
    tp.set_gemm_tile_policy(policy)
    try:
        _graph_step(dtype, n, d, m, t)
    finally:
        tp.set_gemm_tile_policy(tp.GEMM_TILE_AUTO)


def _graph_step(dtype, n, d, m, t):
    sets = []
    for seed in (21, 22, 23):
        inp = mlp_inputs(n, d, m, t, dtype=dtype, seed=seed)
        X, A, B, G = (dev(inp[k]) for k in "XABG")
        sets.append((X, shard_cols(A, t), shard_rows(B, t), G))

    # eager reference of every input set
    ref = []
    for X, A, B, G in sets:
        o = _buffers(X, A, B)
        _step(X, A, B, G, o)
        torch.cuda.synchronize()
        ref.append({k: o[k].clone() for k in OUTS})

    # static inputs and outputs of the graph
    sX, sA, sB, sG = (x.clone() for x in sets[0])
    out = _buffers(sX, sA, sB)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        _step(sX, sA, sB, sG, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(sX, sA, sB, sG, out)
    torch.cuda.synchronize()

    for rep, k in enumerate((1, 2, 0, 1)):
        X, A, B, G = sets[k]
        sX.copy_(X)
        sA.copy_(A)
        sB.copy_(B)
        sG.copy_(G)
        for v in out.values():  # stale results must not survive a replay
            v.fill_(0)
        # eager work on the same stream between replays
        scratch = (X.float() * 2).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for name in OUTS:
            assert torch.equal(out[name], ref[k][name]), f"replay {rep} (input set {k}): {name} differs"


def _graph_check(step, sets, order=(1, 2, 0, 1)):
    """Capture step(*static inputs) (it returns a dict of output tensors, allocated in
    the graph's pool) and replay it on each input set of `order`, comparing bit for bit
    with step(*set) run eagerly."""
    ref = []
    for args in sets:
        out = step(*args)
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in out.items()})
    static = [a.clone() for a in sets[0]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(*static)
    torch.cuda.synchronize()
    for rep, k in enumerate(order):
        for dst, src in zip(static, sets[k]):
            dst.copy_(src)
        for v in out.values():
            v.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, v in out.items():
            assert torch.equal(v, ref[k][name]), f"replay {rep} (input set {k}): {name} differs"


@pytest.mark.parametrize("masked,shape", [
    (False, (130, 2, 256, 2, 2)), (True, (130, 2, 256, 2, 2)),
    # 512 key blocks of 128 with dh 128: the persistent dk/dv kernel is captured
    (False, (256, 16, 2048, 16, 1)),
])
def test_attention_layer_graph(masked, shape):
    s, b, d, heads, t = shape
    dh = d // heads
    say(f"[gpu] graph capture attention s={s} b={b} d={d} heads={heads} t={t} masked={masked}")
    sets = []
    for seed in (31, 32, 33):
        inp = attn_inputs(s, b, d, heads, dtype="bf16", seed=seed, x_std=1.0, w_std=1.2 / np.sqrt(d), g_std=1.0)
        X, Wq, Wp, G = (dev(inp[k]) for k in ("X", "Wqkv", "Wproj", "G"))
        m = torch.from_numpy(attn_mask(b, s, "padding", seed=seed)).cuda() if masked else None
        args = [X, shard_cols(Wq, t), shard_rows(Wp, t), G] + ([m] if masked else [])
        sets.append(args)

    def step(X, Wq, Wp, G, m=None):
        QKV, O, lse, P = tp.attn_fwd(X, Wq, Wp, s, b, dh, not masked, mask=m)
        Out = tp.reduce_partials(P)
        dO, dQKV, dWqkv, dWproj, dXp = tp.attn_bwd(X, Wq, Wp, QKV, O, lse, G, s, b, dh, not masked, mask=m)
        dX = tp.reduce_partials(dXp)
        return dict(QKV=QKV, O=O, lse=lse, Out=Out, dQKV=dQKV, dWqkv=dWqkv, dWproj=dWproj, dX=dX)

    _graph_check(step, sets)


def test_vocab_ce_graph():
    n, h, V, t = 300, 264, 2064, 2
    say(f"[gpu] graph capture vocab CE n={n} h={h} V={V} t={t}")
    sets = []
    for seed in (41, 42, 43):
        inp = vocab_inputs(n, h, V, dtype="bf16", seed=seed, x_std=1.0, w_std=1.2 / np.sqrt(h), g_std=1.0)
        X, W = dev(inp["X"]), dev(inp["W"])
        tg = torch.from_numpy(inp["targets"]).cuda()
        g = torch.from_numpy(inp["g"].f32.copy()).cuda()
        sets.append([X, W.reshape(t, V // t, h).contiguous(), tg, g])

    def step(X, W, tg, g):
        logits, loss, rmax, rsum = tp.vocab_ce_fwd(X, W, tg)
        dlogits, dW, dXp = tp.vocab_ce_bwd(X, W, tg, logits, rmax, rsum, g)
        dX = tp.reduce_partials(dXp)
        return dict(logits=logits, loss=loss, rmax=rmax, rsum=rsum, dlogits=dlogits, dW=dW, dX=dX)

    _graph_check(step, sets)
