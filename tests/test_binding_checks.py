"""The Python binding checks every tensor an entry point reads or writes (shape,
dtype, device) before it calls the library: the C side receives bare pointers
and could not notice a wrongly sized buffer.  Runs on the CPU: with every
tensor right, the only complaint left is that the tensors are not on a GPU;
with one tensor of a wrong shape or dtype, that tensor is named first."""

import pytest
import torch

import megatron_tensor_transformer_amd as tp

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def e(shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def mlp_fwd_args(n=16, d=24, mi=8, t=2):
    return dict(X=e((n, d)), A=e((t, d, mi)), B=e((t, mi, d)), Z=e((t, n, mi)), Y=e((t, n, mi)), P=e((t, n, d)))


def mlp_bwd_args(n=16, d=24, mi=8, t=2):
    a = mlp_fwd_args(n, d, mi, t)
    del a["P"]
    a.update(G=e((n, d)), D=e((t, n, mi)), dA=e((t, d, mi), f32), dB=e((t, mi, d), f32), dXp=e((t, n, d)))
    return a


def attn_fwd_args(s=8, b=2, d=32, heads=2, dh=64, t=2):
    n, w = s * b, heads * dh
    return dict(X=e((n, d)), Wqkv=e((t, d, 3 * w)), Wproj=e((t, w, d)), QKV=e((t, n, 3 * w)), O=e((t, n, w)),
                lse=e((t, b, heads, s), f32), P=e((t, n, d)))


def attn_bwd_args(s=8, b=2, d=32, heads=2, dh=64, t=2):
    a = attn_fwd_args(s, b, d, heads, dh, t)
    n, w = s * b, heads * dh
    del a["P"]
    a.update(G=e((n, d)), dO=e((t, n, w)), dQKV=e((t, n, 3 * w)), dWqkv=e((t, d, 3 * w), f32),
             dWproj=e((t, w, d), f32), dXp=e((t, n, d)), ws=e((64,), torch.uint8))
    return a


def vocab_fwd_args(n=16, h=32, vi=24, t=2):
    return dict(X=e((n, h)), W=e((t, vi, h)), targets=e((n,), i32), logits=e((t, n, vi)), loss=e((n,), f32),
                row_max=e((n,), f32), row_sum=e((n,), f32), ws=e((64,), torch.uint8))


def vocab_bwd_args(n=16, h=32, vi=24, t=2):
    a = vocab_fwd_args(n, h, vi, t)
    del a["loss"], a["ws"]
    a.update(g=e((n,), f32), dlogits=e((t, n, vi)), dW=e((t, vi, h), f32), dXp=e((t, n, h)))
    return a


CASES = {
    "tpmlp_fwd": (tp.tpmlp_fwd, mlp_fwd_args, {}),
    "tpmlp_fwd_bias": (tp.tpmlp_fwd_bias, lambda: {**mlp_fwd_args(), "b1": e((2, 8))}, {}),
    "tpmlp_bwd": (tp.tpmlp_bwd, mlp_bwd_args, {}),
    "tpmlp_bwd_bias": (tp.tpmlp_bwd_bias, lambda: {**mlp_bwd_args(), "db1": e((2, 8), f32), "db2": e((24,), f32)},
                       {}),
    "tpmlp_reduce_partials": (tp.tpmlp_reduce_partials, lambda: dict(partials=e((3, 16, 24)), out=e((16, 24), f32)),
                              {}),
    "tpmlp_reduce_partials_bias": (tp.tpmlp_reduce_partials_bias,
                                   lambda: dict(partials=e((3, 16, 24)), bias=e((24,)), out=e((16, 24))), {}),
    "tpmlp_bias_grad": (tp.tpmlp_bias_grad, lambda: dict(g=e((2, 40, 24)), db=e((2, 24), f32)), {}),
    "tpmlp_attn_fwd": (tp.tpmlp_attn_fwd, attn_fwd_args, dict(s=8, b=2, head_dim=64, causal=True)),
    "tpmlp_attn_fwd_bias": (tp.tpmlp_attn_fwd_bias, lambda: {**attn_fwd_args(), "bqkv": e((2, 384))},
                            dict(s=8, b=2, head_dim=64, causal=True)),
    "tpmlp_attn_bwd": (tp.tpmlp_attn_bwd, attn_bwd_args, dict(s=8, b=2, head_dim=64, causal=True)),
    "tpmlp_attn_core_fwd": (tp.tpmlp_attn_core_fwd,
                            lambda: dict(qkv=e((2, 16, 384)), o=e((2, 16, 128)), lse=e((2, 2, 2, 8), f32)),
                            dict(s=8, b=2, heads=2, head_dim=64, causal=False)),
    "tpmlp_attn_core_bwd": (tp.tpmlp_attn_core_bwd,
                            lambda: dict(qkv=e((2, 16, 384)), o=e((2, 16, 128)), lse=e((2, 2, 2, 8), f32),
                                         d_o=e((2, 16, 128)), dqkv=e((2, 16, 384)), ws=e((64,), torch.uint8)),
                            dict(s=8, b=2, heads=2, head_dim=64, causal=False)),
    "tpmlp_attn_pack_mask": (tp.tpmlp_attn_pack_mask,
                             lambda: dict(mask=e((2, 40, 40), torch.uint8), packed=e((2, 2, 40, 2), i32)), {}),
    "tpmlp_vocab_ce_fwd": (tp.tpmlp_vocab_ce_fwd, vocab_fwd_args, {}),
    "tpmlp_vocab_ce_bwd": (tp.tpmlp_vocab_ce_bwd, vocab_bwd_args, {}),
}

# the tensor that fixes the path dtype and the device: changing it changes
# what the others are checked against
ANCHORS = {"X", "partials", "g", "qkv", "mask"}
SIZE_ANCHORS = {"A", "W", "Wqkv"}


def other_dtype(t):
    return {bf: f32, f32: bf, i32: torch.int64, torch.uint8: torch.int16}[t.dtype]


def expect(status, fn, kwargs, word=None):
    with pytest.raises(tp.TpmlpValueError) as ei:
        fn(**kwargs)
    assert ei.value.status == status, str(ei.value)
    if word is not None:
        assert word in str(ei.value), str(ei.value)


@pytest.mark.parametrize("name", sorted(CASES))
def test_right_tensors_pass_the_checks(name):
    fn, args, extra = CASES[name]
    expect(tp.ERR_ARG, fn, {**args(), **extra}, "not on a GPU")


def _mutable(name):
    fn, args, extra = CASES[name]
    return [(name, k) for k, v in args().items() if k not in ANCHORS and k != "ws"]


@pytest.mark.parametrize("name,arg", [c for n in sorted(CASES) for c in _mutable(n)])
def test_wrong_shape_is_refused(name, arg):
    fn, args, extra = CASES[name]
    a = args()
    v = a[arg]
    a[arg] = torch.zeros(tuple(v.shape[:-1]) + (v.shape[-1] + 8,), dtype=v.dtype)
    # the weights fix the sizes the other tensors are checked against: a
    # wrong weight shape is refused through whichever tensor disagrees first
    expect(tp.ERR_SHAPE, fn, {**a, **extra}, None if arg in SIZE_ANCHORS else arg)


@pytest.mark.parametrize("name,arg", [c for n in sorted(CASES) for c in _mutable(n)])
def test_wrong_dtype_is_refused(name, arg):
    fn, args, extra = CASES[name]
    a = args()
    if name == "tpmlp_reduce_partials" and arg == "out":
        pytest.skip("out may be bf16 or fp32 independently of the partials")
    a[arg] = a[arg].to(other_dtype(a[arg]))
    # the reduce's output dtype is the bias's: either one is then named
    expect(tp.ERR_DTYPE, fn, {**a, **extra}, None if (name, arg) == ("tpmlp_reduce_partials_bias", "out") else arg)


def test_reduce_output_dtypes_are_free():
    for od in (bf, f32):
        expect(tp.ERR_ARG, tp.tpmlp_reduce_partials, dict(partials=e((2, 4, 8)), out=e((4, 8), od)), "not on a GPU")


def test_sp_wrappers_check_their_inputs():
    x = e((16, 24))
    with pytest.raises(tp.TpmlpValueError) as ei:
        tp.sp_ln_fwd(x, e((16,)), e((24,)), 2)
    assert ei.value.status == tp.ERR_SHAPE and "gamma" in str(ei.value)
    with pytest.raises(tp.TpmlpValueError) as ei:
        tp.sp_dropres_fwd(e((2, 16, 24)), x, 0.1, 0, bias=e((24,), f32))
    assert ei.value.status == tp.ERR_DTYPE and "bias" in str(ei.value)
    with pytest.raises(tp.TpmlpValueError) as ei:
        tp.sp_ln_bwd(e((2, 16, 24)), x, x, e((24,)), e((16,), f32), e((15,), f32))
    assert ei.value.status == tp.ERR_SHAPE and "rstd" in str(ei.value)
