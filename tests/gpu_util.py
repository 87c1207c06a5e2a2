"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
in the library's layouts, running a whole shard step, and comparing with the
oracle."""

import sys

import numpy as np
import torch

import megatron_tensor_transformer_amd as tp


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(T):
    """tpmlp_inputs.Tensor -> device tensor of its storage dtype."""
    if T.dtype == "bf16":
        return torch.from_numpy(T.bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(T.f32)).cuda()


def shard_cols(A, t):
    """A [d, m] -> [t, d, m/t], shard i = column block i."""
    d, m = A.shape
    return A.reshape(d, t, m // t).permute(1, 0, 2).contiguous()


def shard_rows(B, t):
    """B [m, d] -> [t, m/t, d], shard i = row block i."""
    m, d = B.shape
    return B.reshape(t, m // t, d).contiguous()


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def relerr(gpu, ref):
    """Relative Frobenius error ‖gpu − ref‖ / ‖ref‖ in fp64."""
    g = gpu if isinstance(gpu, np.ndarray) else f64(gpu)
    r = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(g.astype(np.float64) - r) / (nr if nr > 0 else 1.0))


def run_step(X, A_s, B_s, G):
    """Forward, local reduce, backward, local reduce on the current stream."""
    Z, Y, P = tp.mlp_fwd(X, A_s, B_s)
    O = tp.reduce_partials(P)
    D, dA, dB, dXp = tp.mlp_bwd(X, A_s, B_s, Z, Y, G)
    dX = tp.reduce_partials(dXp)
    torch.cuda.synchronize()
    return dict(Z=Z, Y=Y, P=P, O=O, D=D, dA=dA, dB=dB, dXp=dXp, dX=dX)
