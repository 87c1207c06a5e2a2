"""One MLP shard step (tpmlp_fwd, tpmlp_reduce_partials, tpmlp_bwd, tpmlp_reduce_partials)
captured into a HIP graph and replayed.

The library only enqueues kernels on the caller's stream: it allocates, clears and
synchronises nothing, so the whole step can be captured once and replayed.  Every replay
reads the inputs as they are at replay time; the kernels are deterministic, so each replay
must reproduce the eager step bit for bit.  Eager work and synchronisations run between
the replays, and the inputs change between them, so a replay that reused stale results or
skipped a node would show.
"""

import pytest
import torch

import megatron_tensor_transformer_amd as tp
from tpmlp_inputs import mlp_inputs

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
    )


def _step(X, A, B, G, o):
    tp.tpmlp_fwd(X, A, B, o["Z"], o["Y"], o["P"])
    tp.tpmlp_reduce_partials(o["P"], o["O"])
    tp.tpmlp_bwd(X, A, B, o["Z"], o["Y"], G, o["D"], o["dA"], o["dB"], o["dXp"], o["ws"])
    tp.tpmlp_reduce_partials(o["dXp"], o["dX"])


@pytest.mark.parametrize("dtype,n,d,m,t", [("bf16", 520, 264, 512, 4), ("f32", 130, 72, 96, 3)])
def test_step_graph_replays_match_eager(dtype, n, d, m, t):
    say(f"[gpu] graph capture {dtype} n={n} d={d} m={m} t={t}")
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
