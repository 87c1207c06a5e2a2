"""The allocation-free bias gradient (tpmlp_bias_grad_noalloc) against the
workspace entry point tpmlp_bias_grad, through the C ABI: same kernels and
fixed summation order, so the results must agree bit for bit.  Two calls in a
row on the library's shared scratch array, the second with a smaller input,
so a stale partial from the first call would show in the second."""

import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp

from gpu_util import say

pytestmark = pytest.mark.gpu


def _g(t, rows, cols, dtype, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return (torch.randn((t, rows, cols), generator=gen, device="cuda") * 0.01).to(dtype)


def _both(g):
    t, rows, cols = g.shape
    ref = tp.bias_grad(g)  # the workspace entry point
    out = torch.full((t, cols), float("nan"), dtype=torch.float32, device="cuda")
    tp.tpmlp_bias_grad_noalloc(g, out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    # first: the 8.3B-shaped layer's db1 (3 MiB of scratch); then a smaller,
    # ragged one (partial 128-row chunk, columns not a multiple of 8)
    for k, (t, rows, cols) in enumerate([(8, 8192, 1536), (3, 300, 44)]):
        say(f"[gpu] bias_grad_noalloc call {k}: t={t} rows={rows} cols={cols} {dtype}")
        g = _g(t, rows, cols, dtype, seed=10 + k)
        ref, out = _both(g)
        assert torch.equal(out, ref), f"call {k}: differs from tpmlp_bias_grad"
        # and both are the column sums (fp64 of the stored values)
        want = g.double().sum(dim=1).cpu().numpy()
        err = np.linalg.norm(out.double().cpu().numpy() - want) / np.linalg.norm(want)
        assert err <= 1e-5, f"call {k}: relative error {err:.2e}"


def test_noalloc_zero_rows_and_limit():
    db = torch.full((2, 16), 7.0, dtype=torch.float32, device="cuda")
    tp.tpmlp_bias_grad_noalloc(torch.empty((2, 0, 16), dtype=torch.bfloat16, device="cuda"), db)
    torch.cuda.synchronize()
    assert torch.equal(db, torch.zeros_like(db))
    # 8 shards × 64 chunks × 8200 columns × 4 B > 16 MiB: refused, nothing enqueued
    g = torch.empty((8, 8192, 8200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tp.TpmlpValueError) as ei:
        tp.tpmlp_bias_grad_noalloc(g, torch.empty((8, 8200), dtype=torch.float32, device="cuda"))
    assert ei.value.status == tp.ERR_SCRATCH
