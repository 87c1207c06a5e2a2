"""Python binding of libtpmlp.so, the MI355X (gfx950) tensor-parallel MLP shard
library.  Argument marshalling only: every step runs in the library's HIP
kernels; torch supplies device memory and the current stream.

The functions named tpmlp_* mirror the C entry points of include/tpmlp.h one to
one; mlp_fwd / mlp_bwd / reduce_partials / sp_* allocate their outputs with
torch and then call them.  A missing library or a non-zero status raises; there
is no fallback path.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtpmlp.so")

F32, BF16 = 0, 1
SP_LN_FWD, SP_DROPRES_FWD, SP_DROPRES_BWD, SP_LN_BWD = 0, 1, 2, 3

ERR_NULLPTR, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_HIP, ERR_WORKSPACE, ERR_ARG = -1, -2, -3, -4, -5, -6, -7
ERR_SCRATCH = -8
NOALLOC_SCRATCH_BYTES = 16 << 20  # TPMLP_NOALLOC_SCRATCH_BYTES


class TpmlpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"tpmlp status {status}: {msg}")
        self.status = status


class TpmlpValueError(ValueError):
    def __init__(self, status, msg):
        super().__init__(f"tpmlp status {status}: {msg}")
        self.status = status


class SpArgs(ctypes.Structure):
    """Mirror of tpmlp_sp_args."""
    _fields_ = [
        ("phase", ctypes.c_int32), ("dt", ctypes.c_int32), ("t", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("s", ctypes.c_int64), ("h", ctypes.c_int64),
        ("row0", ctypes.c_int64), ("eps", ctypes.c_float), ("p_drop", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("x", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("ln_out", ctypes.c_void_p), ("mean", ctypes.c_void_p),
        ("rstd", ctypes.c_void_p), ("partials", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("g_out", ctypes.c_void_p), ("dS", ctypes.c_void_p), ("dU_partials", ctypes.c_void_p),
        ("dx", ctypes.c_void_p), ("dgamma", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("bias", ctypes.c_void_p),
    ]


_lib = None

# exported C symbols and their ctypes signatures
_P, _I, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "tpmlp_fwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I32]),
    "tpmlp_fwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ]),
    "tpmlp_fwd_bias_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I32]),
    "tpmlp_fwd_bias": (_I, [_P, _I, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ]),
    "tpmlp_bwd_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I32]),
    "tpmlp_bwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ]),
    "tpmlp_bwd_bias_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I32]),
    "tpmlp_bwd_bias": (_I, [_P, _I, _I64, _I64, _I64, _I32] + [_P] * 13 + [_SZ]),
    "tpmlp_reduce_partials": (_I, [_P, _I, _I, _I32, _I64, _I64, _P, _P]),
    "tpmlp_reduce_partials_bias": (_I, [_P, _I, _I, _I32, _I64, _I64, _P, _P, _P]),
    "tpmlp_bias_grad_workspace_bytes": (_SZ, [_I32, _I64, _I64]),
    "tpmlp_bias_grad": (_I, [_P, _I, _I32, _I64, _I64, _P, _P, _P, _SZ]),
    "tpmlp_bias_grad_noalloc": (_I, [_P, _I, _I32, _I64, _I64, _P, _P]),
    "tpmlp_sp_workspace_bytes": (_SZ, [_I64, _I64]),
    "tpmlp_attn_fwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _I32, _I32, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "tpmlp_attn_fwd_bias": (_I, [_P, _I, _I64, _I64, _I64, _I32, _I32, _I32, _I] + [_P] * 9),
    "tpmlp_attn_bwd_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I32]),
    "tpmlp_attn_bwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _I32, _I32, _I] + [_P] * 14 + [_SZ]),
    "tpmlp_attn_core_fwd": (_I, [_P, _I, _I32, _I64, _I64, _I32, _I32, _I, _P, _P, _P, _P]),
    "tpmlp_attn_core_bwd": (_I, [_P, _I, _I32, _I64, _I64, _I32, _I32, _I, _P, _P, _P, _P, _P, _P, _P, _SZ]),
    "tpmlp_attn_mask_words": (_SZ, [_I64, _I64]),
    "tpmlp_attn_pack_mask": (_I, [_P, _I64, _I64, _P, _P]),
    "tpmlp_ln_sp": (_I, [_P, ctypes.POINTER(SpArgs)]),
    "tpmlp_vocab_ce_workspace_bytes": (_SZ, [_I32, _I64, _I64]),
    "tpmlp_vocab_ce_fwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _I64] + [_P] * 8 + [_SZ]),
    "tpmlp_vocab_ce_bwd": (_I, [_P, _I, _I64, _I64, _I64, _I32, _I64] + [_P] * 10),
    "tpmlp_status_string": (ctypes.c_char_p, [_I]),
    "tpmlp_last_hip_error": (_I, []),
    "tpmlp_abi_version": (_I, []),
    "tpmlp_set_gemm_tile_policy": (_I, [_I]),
    "tpmlp_gemm_tile_policy": (_I, []),
}


def lib():
    """Load libtpmlp.so (built by megatron_tensor_transformer_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m megatron_tensor_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status == 0:
        return
    msg = lib().tpmlp_status_string(status).decode()
    if status == ERR_HIP:
        raise TpmlpError(status, f"{msg} (hipError {lib().tpmlp_last_hip_error()})")
    raise TpmlpValueError(status, msg)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TpmlpValueError(ERR_DTYPE, f"unsupported dtype {t.dtype}")


def _expect(ref, *specs, final=True):
    """Check every tensor an entry point reads or writes before the library is
    called: the C side receives bare pointers and cannot check extents, so a
    tensor of the wrong shape, dtype or device would be read or written past
    its allocation.  ref is the tensor that fixes the device; each spec is
    (name, tensor, shape, dtype), where a None tensor is skipped (an optional
    argument) and a shape entry of None matches any size.  final: this is the
    entry point's last check, so the common device must also be a GPU."""
    for name, t, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TpmlpValueError(ERR_ARG, f"{name} is not a tensor")
        if t.device != ref.device:
            raise TpmlpValueError(ERR_ARG, f"{name} is on {t.device}, expected {ref.device}")
        if dtype is not None and t.dtype != dtype:
            raise TpmlpValueError(ERR_DTYPE, f"{name} has dtype {t.dtype}, expected {dtype}")
        if shape is not None:
            if t.dim() != len(shape) or any(e is not None and int(a) != int(e) for a, e in zip(t.shape, shape)):
                want = tuple("*" if e is None else int(e) for e in shape)
                raise TpmlpValueError(ERR_SHAPE, f"{name} has shape {tuple(t.shape)}, expected {want}")
    if final and not ref.is_cuda:
        raise TpmlpValueError(ERR_ARG, "tensor is not on a GPU")


def _path_dtype(X):
    """The path dtype of an entry point, from its first activation operand."""
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TpmlpValueError(ERR_DTYPE, f"unsupported dtype {X.dtype}")
    return X.dtype


def _dims(name, t, nd):
    if not isinstance(t, torch.Tensor) or t.dim() != nd:
        raise TpmlpValueError(ERR_SHAPE, f"{name} must be a {nd}-d tensor")
    return tuple(int(x) for x in t.shape)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise TpmlpValueError(ERR_ARG, "tensor is not on a GPU")
    if not t.is_contiguous():
        raise TpmlpValueError(ERR_ARG, "tensor is not contiguous")
    return t.data_ptr() or None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---------------------------------------------------------------- raw entry points
def _mlp_fwd_check(X, A, B, Z, Y, P, b1=None):
    t, d, mi = _dims("A", A, 3)
    n = _dims("X", X, 2)[0]
    dt = _path_dtype(X)
    _expect(X, ("X", X, (n, d), dt), ("A", A, (t, d, mi), dt), ("B", B, (t, mi, d), dt),
            ("b1", b1, (t, mi), dt), ("Z", Z, (t, n, mi), dt), ("Y", Y, (t, n, mi), dt), ("P", P, (t, n, d), dt))
    return t, d, mi, n


def tpmlp_fwd(X, A, B, Z, Y, P, ws=None, stream=None):
    """X [n,d]; A [t,d,m_i]; B [t,m_i,d]; Z, Y [t,n,m_i]; P [t,n,d] (all one dtype);
    ws: a device buffer of at least fwd_workspace_bytes(X, A) bytes (None when that is 0)."""
    t, d, mi, n = _mlp_fwd_check(X, A, B, Z, Y, P)
    _expect(X, ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_fwd(_stream(stream), _dt(X), n, d, mi, t, _ptr(X), _ptr(A), _ptr(B),
                           _ptr(Z), _ptr(Y), _ptr(P), _ptr(ws), ws_bytes))


def tpmlp_fwd_bias(X, A, B, b1, Z, Y, P, ws=None, stream=None):
    """tpmlp_fwd with the column bias b1 [t, m_i] (dtype of X)."""
    if b1 is None:
        raise TpmlpValueError(ERR_NULLPTR, "b1 is required")
    t, d, mi, n = _mlp_fwd_check(X, A, B, Z, Y, P, b1)
    _expect(X, ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_fwd_bias(_stream(stream), _dt(X), n, d, mi, t, _ptr(X), _ptr(A), _ptr(B), _ptr(b1),
                                _ptr(Z), _ptr(Y), _ptr(P), _ptr(ws), ws_bytes))


def tpmlp_bwd(X, A, B, Z, Y, G, D, dA, dB, dXp, ws=None, stream=None):
    """Gradients of t_local shards; dA [t,d,m_i] and dB [t,m_i,d] are fp32."""
    t, d, mi = _dims("A", A, 3)
    n = _dims("X", X, 2)[0]
    dt, f32 = _path_dtype(X), torch.float32
    _expect(X, ("X", X, (n, d), dt), ("A", A, (t, d, mi), dt), ("B", B, (t, mi, d), dt),
            ("Z", Z, (t, n, mi), dt), ("Y", Y, (t, n, mi), dt), ("G", G, (n, d), dt), ("D", D, (t, n, mi), dt),
            ("dA", dA, (t, d, mi), f32), ("dB", dB, (t, mi, d), f32), ("dXp", dXp, (t, n, d), dt),
            ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_bwd(_stream(stream), _dt(X), n, d, mi, t, _ptr(X), _ptr(A), _ptr(B), _ptr(Z),
                           _ptr(Y), _ptr(G), _ptr(D), _ptr(dA), _ptr(dB), _ptr(dXp), _ptr(ws), ws_bytes))


def tpmlp_bwd_bias(X, A, B, Z, Y, G, D, dA, dB, dXp, db1, db2, ws=None, stream=None):
    """tpmlp_bwd plus the bias gradients db1 [t, m_i] = Σ_rows D_i and db2 [d] = Σ_rows G (fp32)."""
    t, d, mi = _dims("A", A, 3)
    n = _dims("X", X, 2)[0]
    dt, f32 = _path_dtype(X), torch.float32
    if db1 is None or db2 is None:
        raise TpmlpValueError(ERR_NULLPTR, "db1 and db2 are required")
    _expect(X, ("X", X, (n, d), dt), ("A", A, (t, d, mi), dt), ("B", B, (t, mi, d), dt),
            ("Z", Z, (t, n, mi), dt), ("Y", Y, (t, n, mi), dt), ("G", G, (n, d), dt), ("D", D, (t, n, mi), dt),
            ("dA", dA, (t, d, mi), f32), ("dB", dB, (t, mi, d), f32), ("dXp", dXp, (t, n, d), dt),
            ("db1", db1, (t, mi), f32), ("db2", db2, (d,), f32), ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_bwd_bias(_stream(stream), _dt(X), n, d, mi, t, _ptr(X), _ptr(A), _ptr(B), _ptr(Z),
                                _ptr(Y), _ptr(G), _ptr(D), _ptr(dA), _ptr(dB), _ptr(dXp), _ptr(db1), _ptr(db2),
                                _ptr(ws), ws_bytes))


def _reduce_check(partials, out, final=True):
    if not isinstance(partials, torch.Tensor) or not isinstance(out, torch.Tensor) or partials.dim() < 2:
        raise TpmlpValueError(ERR_SHAPE, "partials must be [t, rows, ...] and out [rows, ...]")
    _path_dtype(partials)
    _path_dtype(out)
    _expect(partials, ("out", out, tuple(partials.shape[1:]), out.dtype), final=final)


def tpmlp_reduce_partials(partials, out, stream=None):
    """out [rows, cols] = Σ_i partials[i]."""
    _reduce_check(partials, out)
    t = partials.shape[0]
    rows = out.shape[0]
    cols = out.numel() // rows if rows else (out.shape[1] if out.dim() > 1 else 1)
    _check(lib().tpmlp_reduce_partials(_stream(stream), _dt(partials), _dt(out), t, rows, cols,
                                       _ptr(partials), _ptr(out)))


def tpmlp_reduce_partials_bias(partials, bias, out, stream=None):
    """out [rows, cols] = Σ_i partials[i] + bias (bias [cols], dtype of out)."""
    if bias is None:
        raise TpmlpValueError(ERR_NULLPTR, "bias is required")
    _reduce_check(partials, out, final=False)
    t = partials.shape[0]
    rows = out.shape[0]
    cols = out.numel() // rows if rows else (out.shape[1] if out.dim() > 1 else 1)
    _expect(out, ("bias", bias, (cols,), out.dtype))
    _check(lib().tpmlp_reduce_partials_bias(_stream(stream), _dt(partials), _dt(out), t, rows, cols,
                                            _ptr(partials), _ptr(bias), _ptr(out)))


def tpmlp_bias_grad(g, db, ws=None, stream=None):
    """db [t, cols] (fp32) = Σ_rows g [t, rows, cols]."""
    t, rows, cols = _dims("g", g, 3)
    _expect(g, ("g", g, (t, rows, cols), _path_dtype(g)), ("db", db, (t, cols), torch.float32),
            ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_bias_grad(_stream(stream), _dt(g), t, rows, cols, _ptr(g), _ptr(db), _ptr(ws),
                                 ws_bytes))


def tpmlp_bias_grad_noalloc(g, db, stream=None):
    """tpmlp_bias_grad with the library's fixed scratch array instead of a
    workspace: allocates nothing (calls on one GPU must not overlap)."""
    t, rows, cols = _dims("g", g, 3)
    _expect(g, ("g", g, (t, rows, cols), _path_dtype(g)), ("db", db, (t, cols), torch.float32))
    _check(lib().tpmlp_bias_grad_noalloc(_stream(stream), _dt(g), t, rows, cols, _ptr(g), _ptr(db)))


def tpmlp_attn_pack_mask(mask, packed, stream=None):
    """mask [b, s, s] uint8/bool (nonzero hides key j from query i) -> packed
    int32 [2, b, s, ⌈s/32⌉] (the form the attention entry points take)."""
    if mask.dtype not in (torch.uint8, torch.bool) or mask.dim() != 3 or mask.shape[1] != mask.shape[2]:
        raise TpmlpValueError(ERR_ARG, "mask must be uint8 or bool of shape (b, s, s)")
    b, s, _ = mask.shape
    _expect(mask, ("packed", packed, (2, b, s, (s + 31) // 32), torch.int32))
    _check(lib().tpmlp_attn_pack_mask(_stream(stream), b, s, _ptr(mask), _ptr(packed)))


def attn_pack_mask(mask, stream=None):
    """Allocating wrapper: the packed form of a [b, s, s] mask, int32 [2, b, s, ⌈s/32⌉]."""
    b, s = mask.shape[0], mask.shape[1]
    packed = torch.empty((2, b, s, (s + 31) // 32), dtype=torch.int32, device=mask.device)
    tpmlp_attn_pack_mask(mask, packed, stream)
    return packed


def _mask_ptr(mask, s, b, stream):
    """The general attention mask for an entry point: None, a packed int32
    tensor [2, b, s, ⌈s/32⌉] (attn_pack_mask), or a uint8 / bool tensor
    [b, s, s], which is packed here on the call's stream."""
    if mask is None:
        return None, None
    if mask.dtype in (torch.uint8, torch.bool):
        if tuple(mask.shape) != (b, s, s):
            raise TpmlpValueError(ERR_ARG, f"mask must have shape {(b, s, s)}")
        mask = attn_pack_mask(mask, stream)
        if stream is not None:
            mask.record_stream(stream)  # freed only after the call's work on that stream
    if mask.dtype != torch.int32 or tuple(mask.shape) != (2, b, s, (s + 31) // 32):
        raise TpmlpValueError(ERR_ARG, f"packed mask must be int32 of shape {(2, b, s, (s + 31) // 32)}")
    return _ptr(mask), mask


def _attn_fwd_check(X, Wqkv, Wproj, bqkv, QKV, O, lse, P, s, b, head_dim, final=True):
    t, d, w3 = _dims("Wqkv", Wqkv, 3)
    if head_dim <= 0 or w3 % (3 * head_dim):
        raise TpmlpValueError(ERR_SHAPE, f"Wqkv's {w3} columns are not heads of 3·{head_dim}")
    heads = w3 // 3 // head_dim
    n, w = s * b, w3 // 3
    dt = _path_dtype(X)
    _expect(X, ("X", X, (n, d), dt), ("Wqkv", Wqkv, (t, d, w3), dt), ("Wproj", Wproj, (t, w, d), dt),
            ("bqkv", bqkv, (t, w3), dt), ("QKV", QKV, (t, n, w3), dt), ("O", O, (t, n, w), dt),
            ("lse", lse, (t, b, heads, s), torch.float32), ("P", P, (t, n, d), dt), final=final)
    return t, d, heads


def _attn_core_check(qkv, o, lse, d_o, dqkv, s, b, heads, head_dim, final=True):
    t = _dims("qkv", qkv, 3)[0]
    n, w = s * b, heads * head_dim
    dt = _path_dtype(qkv)
    _expect(qkv, ("qkv", qkv, (t, n, 3 * w), dt), ("o", o, (t, n, w), dt),
            ("lse", lse, (t, b, heads, s), torch.float32), ("d_o", d_o, (t, n, w), dt),
            ("dqkv", dqkv, (t, n, 3 * w), dt), final=final)
    return t


def tpmlp_attn_fwd(X, Wqkv, Wproj, QKV, O, lse, P, s, b, head_dim, causal, mask=None, stream=None):
    """X [s·b, d]; Wqkv [t, d, 3w]; Wproj [t, w, d]; QKV [t, s·b, 3w]; O [t, s·b, w];
    lse [t, b, heads, s] fp32; P [t, s·b, d]; w = heads·head_dim; mask None, a
    packed mask (attn_pack_mask) or a [b, s, s] uint8/bool mask."""
    t, d, heads = _attn_fwd_check(X, Wqkv, Wproj, None, QKV, O, lse, P, s, b, head_dim)
    mp, _keep = _mask_ptr(mask, s, b, stream)
    _check(lib().tpmlp_attn_fwd(_stream(stream), _dt(X), s, b, d, heads, head_dim, t, int(causal), mp, _ptr(X),
                                _ptr(Wqkv), _ptr(Wproj), _ptr(QKV), _ptr(O), _ptr(lse), _ptr(P)))


def tpmlp_attn_fwd_bias(X, Wqkv, Wproj, bqkv, QKV, O, lse, P, s, b, head_dim, causal, mask=None, stream=None):
    """tpmlp_attn_fwd with the QKV column bias bqkv [t, 3w] added in the QKV GEMM."""
    if bqkv is None:
        raise TpmlpValueError(ERR_NULLPTR, "bqkv is required")
    t, d, heads = _attn_fwd_check(X, Wqkv, Wproj, bqkv, QKV, O, lse, P, s, b, head_dim)
    mp, _keep = _mask_ptr(mask, s, b, stream)
    _check(lib().tpmlp_attn_fwd_bias(_stream(stream), _dt(X), s, b, d, heads, head_dim, t, int(causal), mp,
                                     _ptr(X), _ptr(Wqkv), _ptr(Wproj), _ptr(bqkv), _ptr(QKV), _ptr(O), _ptr(lse),
                                     _ptr(P)))


def tpmlp_attn_bwd(X, Wqkv, Wproj, QKV, O, lse, G, dO, dQKV, dWqkv, dWproj, dXp, ws, s, b, head_dim, causal,
                   mask=None, stream=None):
    t, d, heads = _attn_fwd_check(X, Wqkv, Wproj, None, QKV, O, lse, None, s, b, head_dim, final=False)
    n, w = s * b, heads * head_dim
    dt, f32 = X.dtype, torch.float32
    _expect(X, ("G", G, (n, d), dt), ("dO", dO, (t, n, w), dt), ("dQKV", dQKV, (t, n, 3 * w), dt),
            ("dWqkv", dWqkv, (t, d, 3 * w), f32), ("dWproj", dWproj, (t, w, d), f32), ("dXp", dXp, (t, n, d), dt),
            ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    mp, _keep = _mask_ptr(mask, s, b, stream)
    _check(lib().tpmlp_attn_bwd(_stream(stream), _dt(X), s, b, d, heads, head_dim, t, int(causal), mp, _ptr(X),
                                _ptr(Wqkv), _ptr(Wproj), _ptr(QKV), _ptr(O), _ptr(lse), _ptr(G), _ptr(dO),
                                _ptr(dQKV), _ptr(dWqkv), _ptr(dWproj), _ptr(dXp), _ptr(ws), ws_bytes))


def tpmlp_attn_core_fwd(qkv, o, lse, s, b, heads, head_dim, causal, mask=None, stream=None):
    """qkv [t, s·b, heads·3·head_dim] -> o [t, s·b, heads·head_dim], lse [t, b, heads, s]."""
    t = _attn_core_check(qkv, o, lse, None, None, s, b, heads, head_dim)
    mp, _keep = _mask_ptr(mask, s, b, stream)
    _check(lib().tpmlp_attn_core_fwd(_stream(stream), _dt(qkv), t, s, b, heads, head_dim, int(causal), mp,
                                     _ptr(qkv), _ptr(o), _ptr(lse)))


def tpmlp_attn_core_bwd(qkv, o, lse, d_o, dqkv, ws, s, b, heads, head_dim, causal, mask=None, stream=None):
    t = _attn_core_check(qkv, o, lse, d_o, dqkv, s, b, heads, head_dim, final=False)
    _expect(qkv, ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    mp, _keep = _mask_ptr(mask, s, b, stream)
    _check(lib().tpmlp_attn_core_bwd(_stream(stream), _dt(qkv), t, s, b, heads, head_dim, int(causal), mp,
                                     _ptr(qkv), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dqkv), _ptr(ws), ws_bytes))


def tpmlp_ln_sp(args, stream=None):
    _check(lib().tpmlp_ln_sp(_stream(stream), ctypes.byref(args)))


# bf16 GEMM tile and schedule policy (process-wide): automatic, 256x256 only,
# 256x192 / 256x128 tiles or a K-split tail wherever available
GEMM_TILE_AUTO, GEMM_TILE_256, GEMM_TILE_192, GEMM_STREAMK, GEMM_TILE_128 = 0, 1, 2, 3, 4


def set_gemm_tile_policy(policy):
    _check(lib().tpmlp_set_gemm_tile_policy(policy))


def gemm_tile_policy():
    return lib().tpmlp_gemm_tile_policy()


# ---------------------------------------------------------------- allocating wrappers
def fwd_workspace_bytes(X, A, bias=False):
    t, d, mi = A.shape
    f = lib().tpmlp_fwd_bias_workspace_bytes if bias else lib().tpmlp_fwd_workspace_bytes
    return f(_dt(X), X.shape[0], d, mi, t)


def workspace(nbytes, device):
    """A device workspace of nbytes (None when 0), as the entry points take it."""
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def mlp_fwd(X, A, B, stream=None):
    t, d, mi = A.shape
    n = X.shape[0]
    Z = torch.empty((t, n, mi), dtype=X.dtype, device=X.device)
    Y = torch.empty_like(Z)
    P = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    tpmlp_fwd(X, A, B, Z, Y, P, workspace(fwd_workspace_bytes(X, A), X.device), stream)
    return Z, Y, P


def mlp_fwd_bias(X, A, B, b1, stream=None):
    t, d, mi = A.shape
    n = X.shape[0]
    Z = torch.empty((t, n, mi), dtype=X.dtype, device=X.device)
    Y = torch.empty_like(Z)
    P = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    tpmlp_fwd_bias(X, A, B, b1, Z, Y, P, workspace(fwd_workspace_bytes(X, A, bias=True), X.device), stream)
    return Z, Y, P


def bwd_workspace_bytes(X, A):
    t, d, mi = A.shape
    return lib().tpmlp_bwd_workspace_bytes(_dt(X), X.shape[0], d, mi, t)


def mlp_bwd(X, A, B, Z, Y, G, stream=None):
    t, d, mi = A.shape
    n = X.shape[0]
    D = torch.empty((t, n, mi), dtype=X.dtype, device=X.device)
    dA = torch.empty((t, d, mi), dtype=torch.float32, device=X.device)
    dB = torch.empty((t, mi, d), dtype=torch.float32, device=X.device)
    dXp = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    nb = bwd_workspace_bytes(X, A)
    ws = torch.empty(nb, dtype=torch.uint8, device=X.device) if nb else None
    tpmlp_bwd(X, A, B, Z, Y, G, D, dA, dB, dXp, ws, stream)
    return D, dA, dB, dXp


def bwd_bias_workspace_bytes(X, A):
    t, d, mi = A.shape
    return lib().tpmlp_bwd_bias_workspace_bytes(_dt(X), X.shape[0], d, mi, t)


def mlp_bwd_bias(X, A, B, Z, Y, G, stream=None):
    """Allocating wrapper: returns D, dA, dB, dXp, db1 [t, m_i], db2 [d] (fp32 gradients)."""
    t, d, mi = A.shape
    n = X.shape[0]
    D = torch.empty((t, n, mi), dtype=X.dtype, device=X.device)
    dA = torch.empty((t, d, mi), dtype=torch.float32, device=X.device)
    dB = torch.empty((t, mi, d), dtype=torch.float32, device=X.device)
    dXp = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    db1 = torch.empty((t, mi), dtype=torch.float32, device=X.device)
    db2 = torch.empty((d,), dtype=torch.float32, device=X.device)
    tpmlp_bwd_bias(X, A, B, Z, Y, G, D, dA, dB, dXp, db1, db2, workspace(bwd_bias_workspace_bytes(X, A), X.device),
                   stream)
    return D, dA, dB, dXp, db1, db2


def reduce_partials(partials, out_dtype=None, stream=None):
    out = torch.empty(partials.shape[1:], dtype=out_dtype or partials.dtype, device=partials.device)
    tpmlp_reduce_partials(partials, out, stream)
    return out


def reduce_partials_bias(partials, bias, stream=None):
    out = torch.empty(partials.shape[1:], dtype=bias.dtype, device=partials.device)
    tpmlp_reduce_partials_bias(partials, bias, out, stream)
    return out


def bias_grad_workspace_bytes(t, rows, cols):
    return lib().tpmlp_bias_grad_workspace_bytes(t, rows, cols)


def bias_grad(g, stream=None):
    """Column sums over the rows of g [t, rows, cols] or [rows, cols] -> fp32 [t, cols] or [cols]."""
    g3 = g if g.dim() == 3 else g.unsqueeze(0)
    t, rows, cols = g3.shape
    db = torch.empty((t, cols), dtype=torch.float32, device=g.device)
    nb = bias_grad_workspace_bytes(t, rows, cols)
    ws = torch.empty(nb, dtype=torch.uint8, device=g.device) if nb else None
    tpmlp_bias_grad(g3, db, ws, stream)
    return db if g.dim() == 3 else db[0]


def sp_ln_fwd(x, gamma, beta, t, eps=1e-5, stream=None):
    s, h = _dims("x", x, 2)
    _expect(x, ("gamma", gamma, (h,), _path_dtype(x)), ("beta", beta, (h,), x.dtype))
    U = torch.empty_like(x)
    mean = torch.empty(s, dtype=torch.float32, device=x.device)
    rstd = torch.empty_like(mean)
    a = SpArgs(phase=SP_LN_FWD, dt=_dt(x), t=t, s=s, h=h, eps=eps, x=_ptr(x), gamma=_ptr(gamma),
               beta=_ptr(beta), ln_out=_ptr(U), mean=_ptr(mean), rstd=_ptr(rstd))
    tpmlp_ln_sp(a, stream)
    return U, mean, rstd


def sp_dropres_fwd(partials, x, p, seed, row0=0, bias=None, stream=None):
    t = _dims("partials", partials, 3)[0]
    s, h = _dims("x", x, 2)
    _expect(x, ("partials", partials, (t, s, h), _path_dtype(x)), ("bias", bias, (h,), x.dtype))
    out = torch.empty_like(x)
    a = SpArgs(phase=SP_DROPRES_FWD, dt=_dt(x), t=t, s=s, h=h, row0=row0, eps=1.0, p_drop=p, seed=seed,
               partials=_ptr(partials), x=_ptr(x), out=_ptr(out), bias=_ptr(bias))
    tpmlp_ln_sp(a, stream)
    return out


def sp_dropres_bwd(g_out, t, p, seed, row0=0, stream=None):
    s, h = _dims("g_out", g_out, 2)
    _path_dtype(g_out)
    dS = torch.empty_like(g_out)
    a = SpArgs(phase=SP_DROPRES_BWD, dt=_dt(g_out), t=t, s=s, h=h, row0=row0, eps=1.0, p_drop=p,
               seed=seed, g_out=_ptr(g_out), dS=_ptr(dS))
    tpmlp_ln_sp(a, stream)
    return dS


def sp_ln_bwd(dU_partials, g_out, x, gamma, mean, rstd, stream=None):
    t = _dims("dU_partials", dU_partials, 3)[0]
    s, h = _dims("x", x, 2)
    dt = _path_dtype(x)
    _expect(x, ("dU_partials", dU_partials, (t, s, h), dt), ("g_out", g_out, (s, h), dt),
            ("gamma", gamma, (h,), dt), ("mean", mean, (s,), torch.float32), ("rstd", rstd, (s,), torch.float32))
    dx = torch.empty_like(x)
    dgamma = torch.empty(h, dtype=torch.float32, device=x.device)
    dbeta = torch.empty_like(dgamma)
    nb = lib().tpmlp_sp_workspace_bytes(s, h)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=x.device)
    a = SpArgs(phase=SP_LN_BWD, dt=_dt(x), t=t, s=s, h=h, eps=1.0, dU_partials=_ptr(dU_partials),
               g_out=_ptr(g_out), x=_ptr(x), gamma=_ptr(gamma), mean=_ptr(mean), rstd=_ptr(rstd),
               dx=_ptr(dx), dgamma=_ptr(dgamma), dbeta=_ptr(dbeta), ws=_ptr(ws), ws_bytes=nb)
    tpmlp_ln_sp(a, stream)
    return dx, dgamma, dbeta


def attn_bwd_workspace_bytes(t, s, b, heads):
    return lib().tpmlp_attn_bwd_workspace_bytes(t, s, b, heads)


def attn_fwd(X, Wqkv, Wproj, s, b, head_dim, causal=True, mask=None, stream=None, bqkv=None):
    """Allocating wrapper: returns QKV, O, lse, P (bqkv [t, 3w]: the QKV bias)."""
    t, d, w3 = Wqkv.shape
    w = w3 // 3
    n = X.shape[0]
    QKV = torch.empty((t, n, w3), dtype=X.dtype, device=X.device)
    O = torch.empty((t, n, w), dtype=X.dtype, device=X.device)
    lse = torch.empty((t, b, w // head_dim, s), dtype=torch.float32, device=X.device)
    P = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    if bqkv is None:
        tpmlp_attn_fwd(X, Wqkv, Wproj, QKV, O, lse, P, s, b, head_dim, causal, mask, stream)
    else:
        tpmlp_attn_fwd_bias(X, Wqkv, Wproj, bqkv, QKV, O, lse, P, s, b, head_dim, causal, mask, stream)
    return QKV, O, lse, P


def attn_bwd(X, Wqkv, Wproj, QKV, O, lse, G, s, b, head_dim, causal=True, mask=None, stream=None):
    """Allocating wrapper: returns dO, dQKV, dWqkv, dWproj, dXp."""
    t, d, w3 = Wqkv.shape
    w = w3 // 3
    n = X.shape[0]
    dO = torch.empty((t, n, w), dtype=X.dtype, device=X.device)
    dQKV = torch.empty((t, n, w3), dtype=X.dtype, device=X.device)
    dWqkv = torch.empty((t, d, w3), dtype=torch.float32, device=X.device)
    dWproj = torch.empty((t, w, d), dtype=torch.float32, device=X.device)
    dXp = torch.empty((t, n, d), dtype=X.dtype, device=X.device)
    nb = attn_bwd_workspace_bytes(t, s, b, w // head_dim)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=X.device)
    tpmlp_attn_bwd(X, Wqkv, Wproj, QKV, O, lse, G, dO, dQKV, dWqkv, dWproj, dXp, ws, s, b, head_dim, causal, mask,
                   stream)
    return dO, dQKV, dWqkv, dWproj, dXp


# ---------------------------------------------------------------- vocabulary-parallel cross-entropy
def _vocab_check(X, W, targets, logits, row_max, row_sum, final=True):
    t, vi, h = _dims("W", W, 3)
    n = _dims("X", X, 2)[0]
    dt, f32 = _path_dtype(X), torch.float32
    _expect(X, ("X", X, (n, h), dt), ("W", W, (t, vi, h), dt), ("targets", targets, (n,), torch.int32),
            ("logits", logits, (t, n, vi), dt), ("row_max", row_max, (n,), f32), ("row_sum", row_sum, (n,), f32),
            final=final)
    return t, vi, h, n


def tpmlp_vocab_ce_fwd(X, W, targets, logits, loss, row_max, row_sum, ws, vocab_start=0, stream=None):
    """X [n,h]; W [t,v_i,h]; targets [n] int32; logits [t,n,v_i]; loss, row_max, row_sum [n] fp32."""
    t, vi, h, n = _vocab_check(X, W, targets, logits, row_max, row_sum, final=False)
    _expect(X, ("loss", loss, (n,), torch.float32), ("ws", ws, None, None))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().tpmlp_vocab_ce_fwd(_stream(stream), _dt(X), n, h, vi, t, vocab_start, _ptr(X), _ptr(W),
                                    _ptr(targets), _ptr(logits), _ptr(loss), _ptr(row_max), _ptr(row_sum),
                                    _ptr(ws), ws_bytes))


def tpmlp_vocab_ce_bwd(X, W, targets, logits, row_max, row_sum, g, dlogits, dW, dXp, vocab_start=0, stream=None):
    t, vi, h, n = _vocab_check(X, W, targets, logits, row_max, row_sum, final=False)
    _expect(X, ("g", g, (n,), torch.float32), ("dlogits", dlogits, (t, n, vi), X.dtype),
            ("dW", dW, (t, vi, h), torch.float32), ("dXp", dXp, (t, n, h), X.dtype))
    _check(lib().tpmlp_vocab_ce_bwd(_stream(stream), _dt(X), n, h, vi, t, vocab_start, _ptr(X), _ptr(W),
                                    _ptr(targets), _ptr(logits), _ptr(row_max), _ptr(row_sum), _ptr(g),
                                    _ptr(dlogits), _ptr(dW), _ptr(dXp)))


def vocab_ce_fwd(X, W, targets, vocab_start=0, stream=None):
    """Allocating wrapper: returns logits, loss, row_max, row_sum."""
    t, vi, h = W.shape
    n = X.shape[0]
    logits = torch.empty((t, n, vi), dtype=X.dtype, device=X.device)
    loss = torch.empty(n, dtype=torch.float32, device=X.device)
    rmax, rsum = torch.empty_like(loss), torch.empty_like(loss)
    nb = lib().tpmlp_vocab_ce_workspace_bytes(t, n, vi)
    ws = torch.empty(max(nb, 8), dtype=torch.uint8, device=X.device)
    tpmlp_vocab_ce_fwd(X, W, targets, logits, loss, rmax, rsum, ws, vocab_start, stream)
    return logits, loss, rmax, rsum


def vocab_ce_bwd(X, W, targets, logits, row_max, row_sum, g, vocab_start=0, stream=None):
    """Allocating wrapper: returns dlogits, dW (fp32), dXp."""
    t, vi, h = W.shape
    n = X.shape[0]
    dlogits = torch.empty_like(logits)
    dW = torch.empty((t, vi, h), dtype=torch.float32, device=X.device)
    dXp = torch.empty((t, n, h), dtype=X.dtype, device=X.device)
    tpmlp_vocab_ce_bwd(X, W, targets, logits, row_max, row_sum, g, dlogits, dW, dXp, vocab_start, stream)
    return dlogits, dW, dXp
