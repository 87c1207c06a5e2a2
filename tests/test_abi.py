"""The C-ABI library loads, exports every function include/tpmlp.h declares, and
rejects invalid arguments with the documented status before touching the GPU.
Runs without a GPU: every call here fails validation, so no kernel is
launched."""

import ctypes
import os
import re
import subprocess

import pytest

import torch

import megatron_tensor_transformer_amd as tp
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tpmlp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(tpmlp_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return tp.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tpmlp_fwd", "tpmlp_bwd", "tpmlp_reduce_partials", "tpmlp_ln_sp", "tpmlp_fwd_bias",
              "tpmlp_reduce_partials_bias", "tpmlp_bias_grad", "tpmlp_bias_grad_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in tp.SIGNATURES, f"binding lacks {name}"


def test_abi_version_and_status_strings(L):
    assert L.tpmlp_abi_version() == 9
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -99):
        assert L.tpmlp_status_string(s)


def _fwd(L, dt=1, n=64, d=64, mi=64, t=2, ptr=0x1000, ws=None, ws_bytes=0):
    p = ctypes.c_void_p(ptr)
    return L.tpmlp_fwd(None, dt, n, d, mi, t, p, p, p, p, p, p, ws, ws_bytes)


def test_fwd_validation(L):
    assert _fwd(L, dt=7) == tp.ERR_DTYPE
    assert _fwd(L, n=-1) == tp.ERR_SHAPE
    assert _fwd(L, d=0) == tp.ERR_SHAPE
    assert _fwd(L, mi=0) == tp.ERR_SHAPE
    assert _fwd(L, t=0) == tp.ERR_SHAPE
    assert _fwd(L, d=12) == tp.ERR_ALIGN          # bf16 rows must be multiples of 8
    assert _fwd(L, mi=20) == tp.ERR_ALIGN
    assert _fwd(L, ptr=0x1008) == tp.ERR_ALIGN     # bf16 needs 16-byte bases
    assert _fwd(L, ptr=0) == tp.ERR_NULLPTR
    assert _fwd(L, n=1 << 20, d=1 << 12) == tp.ERR_SHAPE  # 2^33 bytes per operand
    assert _fwd(L, n=0) == 0                        # empty input: nothing to do
    # fp32 accepts any row length and 4-byte alignment
    assert _fwd(L, dt=0, d=3, mi=5, ptr=0) == tp.ERR_NULLPTR
    assert _fwd(L, dt=0, d=3, mi=5, ptr=0x1002) == tp.ERR_ALIGN


def test_split_k_workspace(L):
    """Shapes whose products leave the GPU idle (few 256×256 tiles, long K)
    need a workspace for their K-split partials; the 8.3B-shaped layer and
    the fp32 path need none.  A missing or short workspace is refused before
    anything is enqueued."""
    fw, bw = L.tpmlp_fwd_workspace_bytes, L.tpmlp_bwd_workspace_bytes
    assert fw(1, 8192, 3072, 1536, 8) == 0 and bw(1, 8192, 3072, 1536, 8) == 0
    assert fw(0, 2048, 1024, 4096, 1) == 0 and bw(0, 2048, 1024, 4096, 1) == 0
    # single-shard layer: P = Y·B has 8×4 tiles over K = 4096 (split in 4),
    # dX in the weight-gradient launch (split in 2): S fp32 planes of n×d each
    assert fw(1, 2048, 1024, 4096, 1) == 4 * 2048 * 1024 * 4
    assert bw(1, 2048, 1024, 4096, 1) == 2 * 2048 * 1024 * 4
    assert L.tpmlp_fwd_bias_workspace_bytes(1, 2048, 1024, 4096, 1) == fw(1, 2048, 1024, 4096, 1)
    need = fw(1, 2048, 1024, 4096, 1)
    assert _fwd(L, n=2048, d=1024, mi=4096, t=1) == tp.ERR_WORKSPACE
    assert _fwd(L, n=2048, d=1024, mi=4096, t=1, ws=ctypes.c_void_p(0x1000), ws_bytes=need - 1) == tp.ERR_WORKSPACE
    assert _fwd(L, n=2048, d=1024, mi=4096, t=1, ws=ctypes.c_void_p(0x1008), ws_bytes=need) == tp.ERR_ALIGN
    p = ctypes.c_void_p(0x1000)
    a = [p] * 10
    assert L.tpmlp_bwd(None, 1, 2048, 1024, 4096, 1, *a, None, 0) == tp.ERR_WORKSPACE


def test_fwd_bias_validation(L):
    p = ctypes.c_void_p(0x1000)

    def call(b1=p, dt=1, n=64, d=64, mi=64, t=2):
        return L.tpmlp_fwd_bias(None, dt, n, d, mi, t, p, p, p, b1, p, p, p, None, 0)
    assert call(b1=None) == tp.ERR_NULLPTR
    assert call(b1=ctypes.c_void_p(0x1008)) == tp.ERR_ALIGN
    assert call(dt=0, b1=ctypes.c_void_p(0x1002)) == tp.ERR_ALIGN
    assert call(mi=20) == tp.ERR_ALIGN
    assert call(n=-1) == tp.ERR_SHAPE
    assert call(n=0, b1=None) == 0  # empty input: nothing to do


def test_reduce_bias_validation(L):
    p = ctypes.c_void_p(0x1000)
    assert L.tpmlp_reduce_partials_bias(None, 1, 1, 8, 16, 16, p, None, p) == tp.ERR_NULLPTR
    assert L.tpmlp_reduce_partials_bias(None, 1, 0, 8, 16, 16, p, ctypes.c_void_p(0x1002), p) == tp.ERR_ALIGN
    assert L.tpmlp_reduce_partials_bias(None, 1, 1, 0, 16, 16, p, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_reduce_partials_bias(None, 1, 1, 8, 0, 16, None, p, None) == 0


def test_bias_grad_validation(L):
    p = ctypes.c_void_p(0x1000)
    # one fp32 [cols] partial per 128-row chunk and shard
    assert L.tpmlp_bias_grad_workspace_bytes(8, 8192, 1536) == 8 * 64 * 1536 * 4
    assert L.tpmlp_bias_grad_workspace_bytes(1, 129, 5) == 2 * 5 * 4
    assert L.tpmlp_bias_grad_workspace_bytes(1, 0, 5) == 0
    need = L.tpmlp_bias_grad_workspace_bytes(2, 300, 64)
    assert L.tpmlp_bias_grad(None, 5, 2, 300, 64, p, p, p, need) == tp.ERR_DTYPE
    assert L.tpmlp_bias_grad(None, 1, 0, 300, 64, p, p, p, need) == tp.ERR_SHAPE
    assert L.tpmlp_bias_grad(None, 1, 2, -1, 64, p, p, p, need) == tp.ERR_SHAPE
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 0, p, p, p, need) == tp.ERR_SHAPE
    assert L.tpmlp_bias_grad(None, 1, 70000, 300, 64, p, p, p, need) == tp.ERR_SHAPE
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, p, None, p, need) == tp.ERR_NULLPTR
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, None, p, p, need) == tp.ERR_NULLPTR
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, p, p, p, need - 4) == tp.ERR_WORKSPACE
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, p, p, None, need) == tp.ERR_WORKSPACE
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, ctypes.c_void_p(0x1001), p, p, need) == tp.ERR_ALIGN
    assert L.tpmlp_bias_grad(None, 1, 2, 300, 64, p, ctypes.c_void_p(0x1002), p, need) == tp.ERR_ALIGN


def test_bias_grad_noalloc_validation(L):
    """Same checks as tpmlp_bias_grad, and inputs whose partials would not fit
    the fixed 16 MiB scratch array are refused before anything runs."""
    p = ctypes.c_void_p(0x1000)
    assert L.tpmlp_bias_grad_noalloc(None, 5, 2, 300, 64, p, p) == tp.ERR_DTYPE
    assert L.tpmlp_bias_grad_noalloc(None, 1, 0, 300, 64, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_bias_grad_noalloc(None, 1, 2, 300, 64, p, None) == tp.ERR_NULLPTR
    assert L.tpmlp_bias_grad_noalloc(None, 1, 2, 300, 64, None, p) == tp.ERR_NULLPTR
    assert L.tpmlp_bias_grad_noalloc(None, 1, 2, 300, 64, ctypes.c_void_p(0x1001), p) == tp.ERR_ALIGN
    # 8 shards, 64 chunks of 128 rows, 8200 columns: 16.8 MB of partials > 16 MiB
    assert L.tpmlp_bias_grad_workspace_bytes(8, 8192, 8200) > tp.NOALLOC_SCRATCH_BYTES
    assert L.tpmlp_bias_grad_noalloc(None, 1, 8, 8192, 8200, p, p) == tp.ERR_SCRATCH
    assert L.tpmlp_bias_grad_workspace_bytes(8, 8192, 8192) == tp.NOALLOC_SCRATCH_BYTES
    assert b"scratch" in L.tpmlp_status_string(tp.ERR_SCRATCH)


def test_attn_validation(L):
    p = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)

    def core(dt=1, t=2, s=64, b=2, nh=2, dh=128, causal=1, qkv=p, o=p, lse=p, mask=None):
        return L.tpmlp_attn_core_fwd(None, dt, t, s, b, nh, dh, causal, mask, qkv, o, lse)
    assert core(dt=4) == tp.ERR_DTYPE
    assert core(dh=96) == tp.ERR_SHAPE            # head_dim 64 or 128
    assert core(b=0) == tp.ERR_SHAPE
    assert core(nh=0) == tp.ERR_SHAPE
    assert core(causal=2) == tp.ERR_ARG
    assert core(qkv=z) == tp.ERR_NULLPTR
    assert core(lse=z) == tp.ERR_NULLPTR
    assert core(o=ctypes.c_void_p(0x1008)) == tp.ERR_ALIGN
    assert core(s=0, qkv=z, o=z, lse=z) == 0     # empty sequence: nothing to do
    assert core(s=1 << 20, b=1 << 10) == tp.ERR_SHAPE
    # a packed general mask: 4-byte aligned, one batch entry's part (s·⌈s/32⌉
    # words) below 2^31 bytes
    assert core(mask=ctypes.c_void_p(0x1002)) == tp.ERR_ALIGN
    assert core(mask=p, s=1 << 17, b=1, nh=1, t=1) == tp.ERR_SHAPE
    assert L.tpmlp_attn_mask_words(8, 1024) == 2 * 8 * 1024 * 32
    assert L.tpmlp_attn_mask_words(3, 33) == 2 * 3 * 33 * 2
    assert L.tpmlp_attn_mask_words(0, 33) == 0
    assert L.tpmlp_attn_pack_mask(None, 0, 64, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_attn_pack_mask(None, 2, -1, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_attn_pack_mask(None, 2, 64, z, p) == tp.ERR_NULLPTR
    assert L.tpmlp_attn_pack_mask(None, 2, 64, p, z) == tp.ERR_NULLPTR
    assert L.tpmlp_attn_pack_mask(None, 2, 64, ctypes.c_void_p(0x1001), ctypes.c_void_p(0x1002)) == tp.ERR_ALIGN
    assert L.tpmlp_attn_pack_mask(None, 2, 0, z, z) == 0
    # the backward's workspace is one fp32 δ per (shard, batch entry, head, row)
    assert L.tpmlp_attn_bwd_workspace_bytes(8, 1024, 8, 3) == 8 * 8 * 3 * 1024 * 4
    need = L.tpmlp_attn_bwd_workspace_bytes(2, 64, 2, 2)
    assert L.tpmlp_attn_core_bwd(None, 1, 2, 64, 2, 2, 64, 1, None, p, p, p, p, p, p, need - 4) == tp.ERR_WORKSPACE
    assert L.tpmlp_attn_core_bwd(None, 1, 2, 64, 2, 2, 64, 1, None, p, p, z, p, p, p, need) == tp.ERR_NULLPTR
    # the layer: d % 8 for bf16, weight-gradient pointers required
    assert L.tpmlp_attn_fwd(None, 1, 64, 2, 36, 2, 64, 2, 1, None, p, p, p, p, p, p, p) == tp.ERR_ALIGN
    assert L.tpmlp_attn_fwd(None, 1, 64, 2, 256, 2, 64, 2, 1, None, p, p, p, p, p, z, p) == tp.ERR_NULLPTR
    # the biased forward: the QKV bias is required and aligned like the weights
    assert L.tpmlp_attn_fwd_bias(None, 1, 64, 2, 256, 2, 64, 2, 1, None, p, p, p, z, p, p, p, p) == tp.ERR_NULLPTR
    assert L.tpmlp_attn_fwd_bias(None, 1, 64, 2, 256, 2, 64, 2, 1, None, p, p, p, ctypes.c_void_p(0x1008), p, p, p,
                                 p) == tp.ERR_ALIGN
    args = [p] * 10
    # X, W_qkv, W_proj, QKV, O, lse, G | dO, dQKV, dW_qkv, dW_proj, dXp, ws, ws_bytes
    assert L.tpmlp_attn_bwd(None, 1, 64, 2, 256, 2, 64, 2, 1, None, *args[:7], p, p, z, p, p, p,
                            need) == tp.ERR_NULLPTR
    assert L.tpmlp_attn_bwd(None, 1, 64, 2, 256, 2, 64, 2, 1, None, *args[:7], p, p, p, p, p, None,
                            0) == tp.ERR_WORKSPACE


def test_vocab_ce_validation(L):
    p = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)
    # a pair of fp32 (max, sum) per shard, token and 64 vocabulary columns
    assert L.tpmlp_vocab_ce_workspace_bytes(8, 8192, 6400) == 2 * 8 * 8192 * 100 * 4
    assert L.tpmlp_vocab_ce_workspace_bytes(3, 5, 65) == 2 * 3 * 5 * 2 * 4
    assert L.tpmlp_vocab_ce_workspace_bytes(3, 5, 0) == 0
    need = L.tpmlp_vocab_ce_workspace_bytes(2, 64, 64)

    def fwd(dt=1, n=64, h=64, vi=64, t=2, start=0, X=p, tg=p, ws=p, nb=need):
        return L.tpmlp_vocab_ce_fwd(None, dt, n, h, vi, t, start, X, p, tg, p, p, p, p, ws, nb)
    assert fwd(dt=3) == tp.ERR_DTYPE
    assert fwd(vi=0) == tp.ERR_SHAPE
    assert fwd(vi=12) == tp.ERR_ALIGN
    assert fwd(start=-1) == tp.ERR_ARG
    assert fwd(X=z) == tp.ERR_NULLPTR
    assert fwd(tg=z) == tp.ERR_NULLPTR
    assert fwd(nb=need - 4) == tp.ERR_WORKSPACE
    assert fwd(ws=z) == tp.ERR_WORKSPACE
    assert fwd(ws=ctypes.c_void_p(0x1004)) == tp.ERR_ALIGN  # pairs of floats: 8-byte aligned
    assert fwd(n=0, X=z, tg=z, ws=z, nb=0) == 0
    # backward: dW required; g required when n > 0
    assert L.tpmlp_vocab_ce_bwd(None, 1, 64, 64, 64, 2, 0, p, p, p, p, p, p, p, p, z, p) == tp.ERR_NULLPTR
    assert L.tpmlp_vocab_ce_bwd(None, 1, 64, 64, 64, 2, 0, p, p, p, p, p, p, z, p, p, p) == tp.ERR_NULLPTR


def test_bwd_validation(L):
    p = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)
    args = [p] * 10
    assert L.tpmlp_bwd(None, 3, 64, 64, 64, 2, *args, None, 0) == tp.ERR_DTYPE
    assert L.tpmlp_bwd(None, 1, 64, 60, 64, 2, *args, None, 0) == tp.ERR_ALIGN
    # dA missing
    a = [p] * 10
    a[7] = z
    assert L.tpmlp_bwd(None, 1, 64, 64, 64, 2, *a, None, 0) == tp.ERR_NULLPTR
    a = [p] * 10
    a[6] = z  # D missing
    assert L.tpmlp_bwd(None, 1, 64, 64, 64, 2, *a, None, 0) == tp.ERR_NULLPTR
    assert L.tpmlp_bwd_workspace_bytes(1, 8192, 3072, 1536, 8) == 0
    # the bf16 path writes the fp32 weight gradients with 16-byte stores
    for k in (7, 8):  # dA, dB
        a = [p] * 10
        a[k] = ctypes.c_void_p(0x1008)
        assert L.tpmlp_bwd(None, 1, 64, 64, 64, 2, *a, None, 0) == tp.ERR_ALIGN
        a[6] = z  # f32 path: 4-byte alignment suffices, so the next check (D) fails
        assert L.tpmlp_bwd(None, 0, 64, 64, 64, 2, *a, None, 0) == tp.ERR_NULLPTR


def test_bwd_bias_validation(L):
    p = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)
    a = [p] * 10
    need = L.tpmlp_bwd_bias_workspace_bytes(1, 64, 64, 64, 2)
    # the chunk sums of D (2 shards × 1 chunk × 64) and of G (1 chunk × 64), 256-byte aligned regions
    assert need == 512 + 256
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, z, p, p, need) == tp.ERR_NULLPTR
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, p, z, p, need) == tp.ERR_NULLPTR
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, p, p, p, need - 1) == tp.ERR_WORKSPACE
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, p, p, z, 0) == tp.ERR_WORKSPACE
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, ctypes.c_void_p(0x1002), p, p, need) == tp.ERR_ALIGN
    assert L.tpmlp_bwd_bias(None, 3, 64, 64, 64, 2, *a, p, p, p, need) == tp.ERR_DTYPE
    a[6] = z  # D missing
    assert L.tpmlp_bwd_bias(None, 1, 64, 64, 64, 2, *a, p, p, p, need) == tp.ERR_NULLPTR


def test_reduce_validation(L):
    p = ctypes.c_void_p(0x1000)
    assert L.tpmlp_reduce_partials(None, 2, 1, 8, 16, 16, p, p) == tp.ERR_DTYPE
    assert L.tpmlp_reduce_partials(None, 1, 1, 0, 16, 16, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_reduce_partials(None, 1, 1, 8, -1, 16, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_reduce_partials(None, 1, 1, 8, 16, 0, p, p) == tp.ERR_SHAPE
    assert L.tpmlp_reduce_partials(None, 1, 1, 8, 16, 16, None, p) == tp.ERR_NULLPTR
    assert L.tpmlp_reduce_partials(None, 0, 0, 8, 16, 16, ctypes.c_void_p(0x1001), p) == tp.ERR_ALIGN
    assert L.tpmlp_reduce_partials(None, 1, 1, 8, 0, 16, None, None) == 0


def _sp(**kw):
    base = dict(phase=tp.SP_LN_FWD, dt=1, t=8, s=64, h=64, eps=1e-5, p_drop=0.1, seed=0,
                x=0x1000, gamma=0x1000, beta=0x1000, ln_out=0x1000, mean=0x1000, rstd=0x1000)
    base.update(kw)
    return tp.SpArgs(**base)


def test_sp_validation(L):
    call = lambda a: L.tpmlp_ln_sp(None, ctypes.byref(a))
    assert L.tpmlp_ln_sp(None, None) == tp.ERR_NULLPTR
    assert call(_sp(t=1)) == tp.ERR_SHAPE          # SP requires TP > 1
    assert call(_sp(s=60)) == tp.ERR_SHAPE         # s % t
    assert call(_sp(h=4)) == tp.ERR_SHAPE          # h >= 8
    assert call(_sp(h=36)) == tp.ERR_ALIGN         # h % 8 == 0, both dtypes
    assert call(_sp(h=36, dt=0)) == tp.ERR_ALIGN
    # any width that is a multiple of 8 passes the shape checks (the next
    # check, a NULL output, fails instead)
    for h in (4104, 6144, 25600, 40000):
        assert call(_sp(h=h, ln_out=0)) == tp.ERR_NULLPTR
    assert call(_sp(s=1 << 16, h=1 << 15)) == tp.ERR_SHAPE  # 2^32 bytes: over the operand limit
    assert call(_sp(dt=0, x=0x1004)) == tp.ERR_ALIGN       # f32 too needs 16-byte bases
    assert call(_sp(mean=0x1002)) == tp.ERR_ALIGN
    assert call(_sp(phase=9)) == tp.ERR_ARG
    assert call(_sp(p_drop=1.0)) == tp.ERR_ARG
    assert call(_sp(p_drop=-0.1)) == tp.ERR_ARG
    assert call(_sp(eps=0.0)) == tp.ERR_ARG
    assert call(_sp(dt=5)) == tp.ERR_DTYPE
    assert call(_sp(ln_out=0)) == tp.ERR_NULLPTR
    assert call(_sp(x=0x1004)) == tp.ERR_ALIGN
    assert call(_sp(s=0)) == 0
    assert call(_sp(phase=tp.SP_DROPRES_FWD, partials=0x1000, out=0x1000, bias=0x1008)) == tp.ERR_ALIGN
    assert call(_sp(phase=tp.SP_LN_BWD, dU_partials=0x1000, g_out=0x1000, dx=0x1000,
                    dgamma=0x1000, dbeta=0x1000, ws=0x1000, ws_bytes=16)) == tp.ERR_WORKSPACE
    # one [2, h] fp32 slot per LN-backward block: min(s, 512) blocks
    assert L.tpmlp_sp_workspace_bytes(4096, 4096) == 512 * 2 * 4096 * 4
    assert L.tpmlp_sp_workspace_bytes(6, 64) == 6 * 2 * 64 * 4
    # rows wider than 4096: 4096-column slabs share a grid of about 512
    # blocks (h = 25600: 7 slabs, 74 row blocks), plus two row means per row
    assert L.tpmlp_sp_workspace_bytes(4096, 25600) == (74 * 2 * 25600 + 2 * 4096) * 4
    assert L.tpmlp_sp_workspace_bytes(32, 6144) == (32 * 2 * 6144 + 2 * 32) * 4


def test_sp_args_layout_matches_header(tmp_path):
    """The ctypes mirror of tpmlp_sp_args has the C compiler's size and offsets."""
    fields = [f for f, _ in tp.SpArgs._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "tpmlp.h"\nint main(void){\n'
        '  printf("%zu\\n", sizeof(tpmlp_sp_args));\n'
        + "".join(f'  printf("%zu\\n", offsetof(tpmlp_sp_args, {f}));\n' for f in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(prog), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(tp.SpArgs)
    for f, off in zip(fields, out[1:]):
        assert getattr(tp.SpArgs, f).offset == off, f


def test_gemm_tile_policy_knob(L):
    # host-only state: set, read back, reject other values, restore
    assert tp.gemm_tile_policy() == tp.GEMM_TILE_AUTO
    for p in (tp.GEMM_TILE_256, tp.GEMM_TILE_192, tp.GEMM_STREAMK, tp.GEMM_TILE_128, tp.GEMM_TILE_AUTO):
        tp.set_gemm_tile_policy(p)
        assert tp.gemm_tile_policy() == p
    for bad in (-1, 5, 192):
        assert L.tpmlp_set_gemm_tile_policy(bad) == tp.ERR_ARG
    assert tp.gemm_tile_policy() == tp.GEMM_TILE_AUTO


def test_workspace_query_covers_stream_k():
    """With the K-split-tail policy the forward's workspace query asks for the
    tail's partial tiles: n = 4352, d = m_i = 4096 gives both GEMMs 17 × 16 =
    272 tiles (one round of 256 and 16 more), K = 4096 (64 steps), so the 16
    tail tiles run as 16 pieces each, 256 partial tiles of 256 KiB; without
    the tail neither GEMM needs a workspace."""
    X = torch.empty((4352, 4096), dtype=torch.bfloat16)
    A = torch.empty((1, 4096, 4096), dtype=torch.bfloat16)
    try:
        tp.set_gemm_tile_policy(tp.GEMM_TILE_256)
        plain = tp.fwd_workspace_bytes(X, A)
        tp.set_gemm_tile_policy(tp.GEMM_STREAMK)
        sk = tp.fwd_workspace_bytes(X, A)
    finally:
        tp.set_gemm_tile_policy(tp.GEMM_TILE_AUTO)
    assert plain == 0
    assert sk == 16 * 16 * 256 * 256 * 4
