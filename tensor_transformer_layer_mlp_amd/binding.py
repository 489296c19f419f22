"""ctypes binding of libtpshard.so: the C ABI's entry points under the same names.

Marshalling only.  Each function takes torch CUDA tensors (contiguous, all of one dtype: bfloat16 or
float32), passes their device pointers and the current torch stream to the library, and raises
TpError on a negative status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback of any kind.  Outputs and workspaces are caller-allocated tensors.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TPSHARD_LIB may name another build of the same library (the host-sanitized one for CPU tests)
LIB_PATH = os.environ.get("TPSHARD_LIB") or os.path.join(_HERE, "libtpshard.so")

TP_BF16, TP_F32 = 0, 1
TP_GELU, TP_GELU_TANH = 0, 1
TP_FP8_E4M3, TP_FP8_E5M2 = 0, 1
TP_FP8_EPI_NONE, TP_FP8_EPI_GELU, TP_FP8_EPI_GELU_TANH, TP_FP8_EPI_DGELU, TP_FP8_EPI_DGELU_TANH = 0, 1, 2, 3, 4
STATUS = {0: "TP_OK", -1: "TP_EINVAL", -2: "TP_ENULL", -3: "TP_EALIGN", -4: "TP_EUNSUPPORTED",
          -5: "TP_EWORKSPACE", -6: "TP_EHIP"}

_I, _P, _Z, _F = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
_SIGNATURES = {
    "tp_shard_range": (_I, [_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "tp_qkv_shard_fwd": (_I, [_I] * 7 + [_P] * 4 + [_P]),
    "tp_attn_heads_fwd": (_I, [_I] * 7 + [_P] * 3 + [_P]),
    "tp_mlp_shard_fwd": (_I, [_I] * 6 + [_P] * 8 + [_P]),
    "tp_mlp_shard_bwd": (_I, [_I] * 6 + [_P] * 11 + [_P, _Z, _P]),
    "tp_mlp_shard_fwd_act": (_I, [_I] * 6 + [_P] * 8 + [_I, _P]),
    "tp_mlp_shard_bwd_act": (_I, [_I] * 6 + [_P] * 11 + [_P, _Z, _I, _P]),
    "tp_qkv_shard_bwd": (_I, [_I] * 7 + [_P] * 6 + [_P, _Z, _P]),
    "tp_qkv_shard_bwd_noalloc": (_I, [_I] * 7 + [_P] * 6 + [_P]),
    "tp_qkv_shard_bwd_noalloc_max_scratch": (_Z, []),
    "tp_attn_heads_bwd": (_I, [_I] * 7 + [_P] * 5 + [_P, _Z, _P]),
    "tp_attn_out_shard_fwd": (_I, [_I] * 7 + [_P] * 4 + [_P]),
    "tp_attn_out_shard_bwd": (_I, [_I] * 7 + [_P] * 6 + [_P, _Z, _P]),
    "tp_residual_ln_fwd": (_I, [_I] * 6 + [_P, _P, _P, _F, _P, _P, _F, _P, _P, _P, _P, _P]),
    "tp_residual_ln_bwd": (_I, [_I] * 6 + [_P] * 7 + [_F] + [_P] * 4 + [_P, _Z, _P]),
    "tp_mlp_grouped_shard_fwd": (_I, [_I, _I, _I, _P, _I, _I, _I, _I] + [_P] * 7 + [_P, _Z, _P]),
    "tp_moe_route": (_I, [_I, _I, _I] + [_P] * 6 + [_P, _Z, _P]),
    "tp_fp8_quantize": (_I, [_I, _I, _I, _P, _I, _P, _P, _P, _P, _Z, _P]),
    "tp_fp8_gemm_nt": (_I, [_I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P]),
    "tp_bias_grad": (_I, [_I, _I, _I, _P, _P, _P, _Z, _P]),
    "tp_mlp_grouped_shard_bwd": (_I, [_I, _I, _I, _P, _I, _I, _I, _I] + [_P] * 10 + [_P, _Z, _P]),
    "tp_moe_shard_bwd": (_I, [_I] * 8 + [_P] * 16 + [_P, _Z, _P]),
    "tp_moe_route_bwd": (_I, [_I, _I, _I, _P, _P, _P, _P, _P]),
    "tp_moe_shard_fwd": (_I, [_I] * 8 + [_P] * 12 + [_P, _Z, _P]),
    "tp_workspace_bytes": (_Z, [ctypes.c_char_p] + [_I] * 8),
    "tp_status_str": (ctypes.c_char_p, [_I]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_version": (ctypes.c_char_p, []),
    "tp_prof_enable": (_I, [_I]),
    "tp_prof_collect": (_I, [_I, ctypes.c_char_p, _I, ctypes.POINTER(_I)] + [ctypes.POINTER(ctypes.c_double)] * 3),
}
ENTRY_POINTS = tuple(_SIGNATURES)

_lib = None


class TpError(RuntimeError):
    def __init__(self, status, fn, detail):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} {detail}")


def raw():
    """The loaded ctypes library (loaded on first use; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_transformer_layer_mlp_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(rc, fn):
    if rc != 0:
        raise TpError(rc, fn, raw().tp_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _need(t, n, name):
    """The library takes raw pointers and cannot see buffer sizes: refuse a tensor with fewer
    elements than the call will touch, before anything is launched."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, the call needs {n}")


def _heads(tp_size, rank, H, n_heads):
    """(heads on this rank, head width) when the geometry is well formed, else None (the library
    then rejects the call with its own message)."""
    if not (1 <= tp_size and 0 <= rank < tp_size and n_heads >= tp_size and H >= 1 and H % n_heads == 0):
        return None
    return tp_shard_range(n_heads, tp_size, rank)[1], H // n_heads


def _cols(tp_size, rank, F):
    if not (1 <= tp_size and 0 <= rank < tp_size and F >= tp_size):
        return None
    return tp_shard_range(F, tp_size, rank)[1]


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def tp_shard_range(n, tp_size, rank):
    off, cnt = _I(), _I()
    _check(raw().tp_shard_range(n, tp_size, rank, ctypes.byref(off), ctypes.byref(cnt)), "tp_shard_range")
    return off.value, cnt.value


def tp_workspace_bytes(fn, tp_size, rank, B, S, H, n_heads, F, dtype):
    code = dtype if isinstance(dtype, int) else (TP_BF16 if dtype == torch.bfloat16 else TP_F32)
    return raw().tp_workspace_bytes(fn.encode(), tp_size, rank, B, S, H, n_heads, F, code)


def tp_qkv_shard_fwd(tp_size, rank, B, S, H, n_heads, X, Wqkv_r, bqkv_r, QKV_r, stream=None):
    dt = X.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, Nq = B * S, 3 * g[0] * g[1]
        for t, n, name in ((X, T * H, "X"), (Wqkv_r, H * Nq, "Wqkv_r"), (bqkv_r, Nq, "bqkv_r"), (QKV_r, T * Nq, "QKV_r")):
            _need(t, n, name)
    rc = raw().tp_qkv_shard_fwd(tp_size, rank, B, S, H, n_heads, _dtype_code(X), _ptr(X, "X", dt),
                                _ptr(Wqkv_r, "Wqkv_r", dt), _ptr(bqkv_r, "bqkv_r", dt),
                                _ptr(QKV_r, "QKV_r", dt), _stream(stream))
    _check(rc, "tp_qkv_shard_fwd")


def tp_attn_heads_fwd(tp_size, rank, B, S, H, n_heads, QKV_r, ctx_r, lse_r=None, stream=None):
    dt = QKV_r.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, nh, d = B * S, g[0], g[1]
        for t, n, name in ((QKV_r, T * 3 * nh * d, "QKV_r"), (ctx_r, T * nh * d, "ctx_r"), (lse_r, B * nh * S, "lse_r")):
            _need(t, n, name)
    rc = raw().tp_attn_heads_fwd(tp_size, rank, B, S, H, n_heads, _dtype_code(QKV_r),
                                 _ptr(QKV_r, "QKV_r", dt), _ptr(ctx_r, "ctx_r", dt),
                                 _ptr(lse_r, "lse_r", torch.float32, True), _stream(stream))
    _check(rc, "tp_attn_heads_fwd")


def tp_mlp_shard_fwd(tp_size, rank, T, H, F, X, W1_r, b1_r, W2_r, b2, Z_r, A1_r, Y_r, stream=None, activation=None):
    dt = X.dtype
    Fr = _cols(tp_size, rank, F)
    if Fr and T >= 0 and H >= 1:
        for t, n, name in ((X, T * H, "X"), (W1_r, H * Fr, "W1_r"), (b1_r, Fr, "b1_r"), (W2_r, Fr * H, "W2_r"),
                           (b2, H, "b2"), (Z_r, T * H, "Z_r"), (A1_r, T * Fr, "A1_r"), (Y_r, T * Fr, "Y_r")):
            _need(t, n, name)
    args = (tp_size, rank, T, H, F, _dtype_code(X), _ptr(X, "X", dt), _ptr(W1_r, "W1_r", dt), _ptr(b1_r, "b1_r", dt),
            _ptr(W2_r, "W2_r", dt), _ptr(b2, "b2", dt, True), _ptr(Z_r, "Z_r", dt), _ptr(A1_r, "A1_r", dt, True),
            _ptr(Y_r, "Y_r", dt))
    if activation is None:      # the plain entry point: the exact GeLU
        _check(raw().tp_mlp_shard_fwd(*args, _stream(stream)), "tp_mlp_shard_fwd")
    else:
        _check(raw().tp_mlp_shard_fwd_act(*args, activation, _stream(stream)), "tp_mlp_shard_fwd_act")


def tp_mlp_shard_bwd(tp_size, rank, T, H, F, X, W1_r, W2_r, A1_r, Y_r, dZ, dX_r, dW1_r, db1_r,
                     dW2_r, db2, workspace, stream=None, activation=None):
    dt = X.dtype
    Fr = _cols(tp_size, rank, F)
    if Fr and T >= 0 and H >= 1:
        for t, n, name in ((X, T * H, "X"), (W1_r, H * Fr, "W1_r"), (W2_r, Fr * H, "W2_r"), (A1_r, T * Fr, "A1_r"),
                           (Y_r, T * Fr, "Y_r"), (dZ, T * H, "dZ"), (dX_r, T * H, "dX_r"), (dW1_r, H * Fr, "dW1_r"),
                           (db1_r, Fr, "db1_r"), (dW2_r, Fr * H, "dW2_r"), (db2, H, "db2")):
            _need(t, n, name)
    args = (tp_size, rank, T, H, F, _dtype_code(X), _ptr(X, "X", dt), _ptr(W1_r, "W1_r", dt), _ptr(W2_r, "W2_r", dt),
            _ptr(A1_r, "A1_r", dt), _ptr(Y_r, "Y_r", dt), _ptr(dZ, "dZ", dt), _ptr(dX_r, "dX_r", dt),
            _ptr(dW1_r, "dW1_r", dt), _ptr(db1_r, "db1_r", dt), _ptr(dW2_r, "dW2_r", dt), _ptr(db2, "db2", dt, True),
            _ptr(workspace, "workspace", None, True),
            workspace.numel() * workspace.element_size() if workspace is not None else 0)
    if activation is None:      # the plain entry point: the exact GeLU
        _check(raw().tp_mlp_shard_bwd(*args, _stream(stream)), "tp_mlp_shard_bwd")
    else:
        _check(raw().tp_mlp_shard_bwd_act(*args, activation, _stream(stream)), "tp_mlp_shard_bwd_act")


def tp_qkv_shard_bwd(tp_size, rank, B, S, H, n_heads, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r,
                     workspace, stream=None):
    dt = X.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, Nq = B * S, 3 * g[0] * g[1]
        for t, n, name in ((X, T * H, "X"), (Wqkv_r, H * Nq, "Wqkv_r"), (dQKV_r, T * Nq, "dQKV_r"),
                           (dX_r, T * H, "dX_r"), (dWqkv_r, H * Nq, "dWqkv_r"), (dbqkv_r, Nq, "dbqkv_r")):
            _need(t, n, name)
    rc = raw().tp_qkv_shard_bwd(tp_size, rank, B, S, H, n_heads, _dtype_code(X), _ptr(X, "X", dt),
                                _ptr(Wqkv_r, "Wqkv_r", dt), _ptr(dQKV_r, "dQKV_r", dt),
                                _ptr(dX_r, "dX_r", dt), _ptr(dWqkv_r, "dWqkv_r", dt),
                                _ptr(dbqkv_r, "dbqkv_r", dt), _ptr(workspace, "workspace", None, True),
                                workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                _stream(stream))
    _check(rc, "tp_qkv_shard_bwd")


def tp_qkv_shard_bwd_noalloc(tp_size, rank, B, S, H, n_heads, X, Wqkv_r, dQKV_r, dX_r, dWqkv_r, dbqkv_r,
                             stream=None):
    """tp_qkv_shard_bwd on the library's own scratch array (no workspace argument; allocates nothing)."""
    dt = X.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, Nq = B * S, 3 * g[0] * g[1]
        for t, n, name in ((X, T * H, "X"), (Wqkv_r, H * Nq, "Wqkv_r"), (dQKV_r, T * Nq, "dQKV_r"),
                           (dX_r, T * H, "dX_r"), (dWqkv_r, H * Nq, "dWqkv_r"), (dbqkv_r, Nq, "dbqkv_r")):
            _need(t, n, name)
    rc = raw().tp_qkv_shard_bwd_noalloc(tp_size, rank, B, S, H, n_heads, _dtype_code(X), _ptr(X, "X", dt),
                                        _ptr(Wqkv_r, "Wqkv_r", dt), _ptr(dQKV_r, "dQKV_r", dt),
                                        _ptr(dX_r, "dX_r", dt), _ptr(dWqkv_r, "dWqkv_r", dt),
                                        _ptr(dbqkv_r, "dbqkv_r", dt), _stream(stream))
    _check(rc, "tp_qkv_shard_bwd_noalloc")


def tp_qkv_shard_bwd_noalloc_max_scratch():
    return int(raw().tp_qkv_shard_bwd_noalloc_max_scratch())


def tp_attn_heads_bwd(tp_size, rank, B, S, H, n_heads, QKV_r, ctx_r, lse_r, dctx_r, dQKV_r,
                      workspace, stream=None):
    dt = QKV_r.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, nh, d = B * S, g[0], g[1]
        for t, n, name in ((QKV_r, T * 3 * nh * d, "QKV_r"), (ctx_r, T * nh * d, "ctx_r"), (lse_r, B * nh * S, "lse_r"),
                           (dctx_r, T * nh * d, "dctx_r"), (dQKV_r, T * 3 * nh * d, "dQKV_r")):
            _need(t, n, name)
    rc = raw().tp_attn_heads_bwd(tp_size, rank, B, S, H, n_heads, _dtype_code(QKV_r),
                                 _ptr(QKV_r, "QKV_r", dt), _ptr(ctx_r, "ctx_r", dt),
                                 _ptr(lse_r, "lse_r", torch.float32), _ptr(dctx_r, "dctx_r", dt),
                                 _ptr(dQKV_r, "dQKV_r", dt), _ptr(workspace, "workspace", None, True),
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(stream))
    _check(rc, "tp_attn_heads_bwd")


def tp_attn_out_shard_fwd(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, bo, O_r, stream=None):
    dt = ctx_r.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, Kr = B * S, g[0] * g[1]
        for t, n, name in ((ctx_r, T * Kr, "ctx_r"), (Wo_r, Kr * H, "Wo_r"), (bo, H, "bo"), (O_r, T * H, "O_r")):
            _need(t, n, name)
    rc = raw().tp_attn_out_shard_fwd(tp_size, rank, B, S, H, n_heads, _dtype_code(ctx_r),
                                     _ptr(ctx_r, "ctx_r", dt), _ptr(Wo_r, "Wo_r", dt),
                                     _ptr(bo, "bo", dt, True), _ptr(O_r, "O_r", dt), _stream(stream))
    _check(rc, "tp_attn_out_shard_fwd")


def tp_attn_out_shard_bwd(tp_size, rank, B, S, H, n_heads, ctx_r, Wo_r, dO, dctx_r, dWo_r, dbo,
                          workspace, stream=None):
    dt = ctx_r.dtype
    g = _heads(tp_size, rank, H, n_heads)
    if g and B >= 0 and S >= 0:
        T, Kr = B * S, g[0] * g[1]
        for t, n, name in ((ctx_r, T * Kr, "ctx_r"), (Wo_r, Kr * H, "Wo_r"), (dO, T * H, "dO"),
                           (dctx_r, T * Kr, "dctx_r"), (dWo_r, Kr * H, "dWo_r"), (dbo, H, "dbo")):
            _need(t, n, name)
    rc = raw().tp_attn_out_shard_bwd(tp_size, rank, B, S, H, n_heads, _dtype_code(ctx_r),
                                     _ptr(ctx_r, "ctx_r", dt), _ptr(Wo_r, "Wo_r", dt), _ptr(dO, "dO", dt),
                                     _ptr(dctx_r, "dctx_r", dt), _ptr(dWo_r, "dWo_r", dt),
                                     _ptr(dbo, "dbo", dt, True), _ptr(workspace, "workspace", None, True),
                                     workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                     _stream(stream))
    _check(rc, "tp_attn_out_shard_bwd")


def _ln_rows(tp_size, rank, sequence_parallel, T):
    if not (1 <= tp_size and 0 <= rank < tp_size and T >= 0):
        return None
    return tp_shard_range(T, tp_size, rank)[1] if sequence_parallel else T


def tp_residual_ln_fwd(tp_size, rank, sequence_parallel, T, H, x, o, keep, p_drop, gamma, beta, eps, h, y, mean,
                       rstd, stream=None):
    """Residual add with dropout, then LayerNorm, on the rank's rows (all T, or its sequence block
    when sequence_parallel); keep is a uint8 tensor (non-zero = kept) or None."""
    dt = x.dtype
    rows = _ln_rows(tp_size, rank, sequence_parallel, T)
    if rows is not None and H >= 1:
        n = rows * H
        for t, k, name in ((x, n, "x"), (o, n, "o"), (keep, n, "keep"), (gamma, H, "gamma"), (beta, H, "beta"),
                           (h, n, "h"), (y, n, "y"), (mean, rows, "mean"), (rstd, rows, "rstd")):
            _need(t, k, name)
    rc = raw().tp_residual_ln_fwd(tp_size, rank, 1 if sequence_parallel else 0, T, H, _dtype_code(x),
                                  _ptr(x, "x", dt), _ptr(o, "o", dt, True), _ptr(keep, "keep", torch.uint8, True),
                                  float(p_drop), _ptr(gamma, "gamma", dt), _ptr(beta, "beta", dt), float(eps),
                                  _ptr(h, "h", dt, True), _ptr(y, "y", dt), _ptr(mean, "mean", torch.float32),
                                  _ptr(rstd, "rstd", torch.float32), _stream(stream))
    _check(rc, "tp_residual_ln_fwd")


def tp_residual_ln_bwd(tp_size, rank, sequence_parallel, T, H, dy, dh_in, h, mean, rstd, gamma, keep, p_drop,
                       dh, d_o, dgamma, dbeta, workspace, stream=None):
    dt = dy.dtype
    rows = _ln_rows(tp_size, rank, sequence_parallel, T)
    if rows is not None and H >= 1:
        n = rows * H
        for t, k, name in ((dy, n, "dy"), (dh_in, n, "dh_in"), (h, n, "h"), (mean, rows, "mean"), (rstd, rows, "rstd"),
                           (gamma, H, "gamma"), (keep, n, "keep"), (dh, n, "dh"), (d_o, n, "d_o"),
                           (dgamma, H, "dgamma"), (dbeta, H, "dbeta")):
            _need(t, k, name)
    rc = raw().tp_residual_ln_bwd(tp_size, rank, 1 if sequence_parallel else 0, T, H, _dtype_code(dy),
                                  _ptr(dy, "dy", dt), _ptr(dh_in, "dh_in", dt, True), _ptr(h, "h", dt),
                                  _ptr(mean, "mean", torch.float32), _ptr(rstd, "rstd", torch.float32),
                                  _ptr(gamma, "gamma", dt), _ptr(keep, "keep", torch.uint8, True), float(p_drop),
                                  _ptr(dh, "dh", dt), _ptr(d_o, "d_o", dt, True), _ptr(dgamma, "dgamma", dt),
                                  _ptr(dbeta, "dbeta", dt), _ptr(workspace, "workspace", None, True),
                                  workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                  _stream(stream))
    _check(rc, "tp_residual_ln_bwd")


def tp_mlp_grouped_shard_fwd(tp_size, rank, n_groups, group_offsets, rows, H, F_group, X_perm, W1_r,
                             b1_r, W2_r, Z_r, A1_r, Y_r, workspace, stream=None):
    dt = X_perm.dtype
    Fr = _cols(tp_size, rank, F_group)
    if Fr and rows >= 0 and H >= 1 and n_groups >= 1:
        G = n_groups
        for t, n, name in ((group_offsets, G + 1, "group_offsets"), (X_perm, rows * H, "X_perm"),
                           (W1_r, G * H * Fr, "W1_r"), (b1_r, G * Fr, "b1_r"), (W2_r, G * Fr * H, "W2_r"),
                           (Z_r, rows * H, "Z_r"), (A1_r, rows * Fr, "A1_r"), (Y_r, rows * Fr, "Y_r")):
            _need(t, n, name)
    rc = raw().tp_mlp_grouped_shard_fwd(
        tp_size, rank, n_groups, _ptr(group_offsets, "group_offsets", torch.int32), rows, H, F_group,
        _dtype_code(X_perm), _ptr(X_perm, "X_perm", dt), _ptr(W1_r, "W1_r", dt), _ptr(b1_r, "b1_r", dt),
        _ptr(W2_r, "W2_r", dt), _ptr(Z_r, "Z_r", dt), _ptr(A1_r, "A1_r", dt, True), _ptr(Y_r, "Y_r", dt),
        _ptr(workspace, "workspace", None, True),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream))
    _check(rc, "tp_mlp_grouped_shard_fwd")


def tp_moe_route(tokens, n_experts, top_k, logits, gates, expert_idx, group_offsets, row_token, token_row,
                 workspace, stream=None):
    """Top-k routing and the expert-sorted dispatch order (int32 outputs, fp32 gates)."""
    n = tokens * top_k if tokens >= 0 and top_k >= 1 else 0
    for t, k, name in ((logits, tokens * n_experts, "logits"), (gates, n, "gates"), (expert_idx, n, "expert_idx"),
                       (group_offsets, n_experts + 1, "group_offsets"), (row_token, n, "row_token"),
                       (token_row, n, "token_row")):
        _need(t, k, name)
    rc = raw().tp_moe_route(tokens, n_experts, top_k, _ptr(logits, "logits", torch.float32),
                            _ptr(gates, "gates", torch.float32), _ptr(expert_idx, "expert_idx", torch.int32),
                            _ptr(group_offsets, "group_offsets", torch.int32), _ptr(row_token, "row_token", torch.int32),
                            _ptr(token_row, "token_row", torch.int32), _ptr(workspace, "workspace", None, True),
                            workspace.numel() * workspace.element_size() if workspace is not None else 0,
                            _stream(stream))
    _check(rc, "tp_moe_route")


def tp_moe_shard_fwd(tp_size, rank, tokens, H, n_experts, top_k, F_expert, X, gates, group_offsets, row_token,
                     token_row, W1_r, b1_r, W2_r, out_r, Z_r, A1_r, Y_r, workspace, stream=None):
    dt = X.dtype
    Fr = _cols(tp_size, rank, F_expert)
    if Fr and tokens >= 0 and top_k >= 1 and H >= 1 and n_experts >= 1:
        n, E = tokens * top_k, n_experts
        for t, k, name in ((X, tokens * H, "X"), (gates, n, "gates"), (group_offsets, E + 1, "group_offsets"),
                           (row_token, n, "row_token"), (token_row, n, "token_row"), (W1_r, E * H * Fr, "W1_r"),
                           (b1_r, E * Fr, "b1_r"), (W2_r, E * Fr * H, "W2_r"), (out_r, tokens * H, "out_r"),
                           (Z_r, n * H, "Z_r"), (A1_r, n * Fr, "A1_r"), (Y_r, n * Fr, "Y_r")):
            _need(t, k, name)
    rc = raw().tp_moe_shard_fwd(
        tp_size, rank, tokens, H, n_experts, top_k, F_expert, _dtype_code(X), _ptr(X, "X", dt),
        _ptr(gates, "gates", torch.float32), _ptr(group_offsets, "group_offsets", torch.int32),
        _ptr(row_token, "row_token", torch.int32), _ptr(token_row, "token_row", torch.int32),
        _ptr(W1_r, "W1_r", dt), _ptr(b1_r, "b1_r", dt), _ptr(W2_r, "W2_r", dt), _ptr(out_r, "out_r", dt),
        _ptr(Z_r, "Z_r", dt), _ptr(A1_r, "A1_r", dt, True), _ptr(Y_r, "Y_r", dt),
        _ptr(workspace, "workspace", None, True),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream))
    _check(rc, "tp_moe_shard_fwd")


def tp_fp8_quantize(x, q, descale, workspace, q_t=None, fmt=TP_FP8_E4M3, stream=None):
    """8-bit codes of a 2-D tensor x with one scale: q uint8 [rows, cols] (or None) and / or q_t uint8
    [cols, rows], the transposed copy; descale a one-element fp32 device tensor.  fmt: TP_FP8_E4M3 /
    TP_FP8_E5M2."""
    rows, cols = x.shape
    _need(q, rows * cols, "q")
    _need(q_t, rows * cols, "q_t")
    _need(descale, 1, "descale")
    rc = raw().tp_fp8_quantize(rows, cols, _dtype_code(x), _ptr(x, "x"), fmt, _ptr(q, "q", torch.uint8, True),
                               _ptr(q_t, "q_t", torch.uint8, True), _ptr(descale, "descale", torch.float32),
                               _ptr(workspace, "workspace", None, True),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream))
    _check(rc, "tp_fp8_quantize")


def tp_fp8_gemm_nt(A, a_descale, B, b_descale, C, bias=None, epilogue=TP_FP8_EPI_NONE, aux=None, C_pre=None,
                   a_fmt=TP_FP8_E4M3, b_fmt=TP_FP8_E4M3, stream=None):
    """C [M, N] bf16 = (A·Bᵀ)·descales (+ bias), then the epilogue, for 8-bit codes A [M, K], B [N, K]."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"B has {B.shape[1]} columns, A has {K}")
    for t, k, name in ((C, M * N, "C"), (bias, N, "bias"), (C_pre, M * N, "C_pre"), (aux, M * N, "aux"),
                       (a_descale, 1, "a_descale"), (b_descale, 1, "b_descale")):
        _need(t, k, name)
    rc = raw().tp_fp8_gemm_nt(M, N, K, _ptr(A, "A", torch.uint8), a_fmt, _ptr(a_descale, "a_descale", torch.float32),
                              _ptr(B, "B", torch.uint8), b_fmt, _ptr(b_descale, "b_descale", torch.float32),
                              _ptr(bias, "bias", torch.bfloat16, True), int(epilogue),
                              _ptr(aux, "aux", torch.bfloat16, True), _ptr(C, "C", torch.bfloat16),
                              _ptr(C_pre, "C_pre", torch.bfloat16, True), _stream(stream))
    _check(rc, "tp_fp8_gemm_nt")


def tp_mlp_grouped_shard_bwd(tp_size, rank, group_offsets, H, F_group, X_perm, W1_r, W2_r, A1_r, Y_r, dZ_perm,
                             dX_perm, dW1_r, db1_r, dW2_r, workspace, stream=None):
    """Backward of tp_mlp_grouped_shard_fwd on expert-sorted rows (dX_perm may be dZ_perm)."""
    G = W1_r.shape[0]
    rows = X_perm.shape[0]
    _, Fr = tp_shard_range(F_group, tp_size, rank) if 0 <= rank < tp_size and F_group >= tp_size >= 1 else (0, 0)
    _need(group_offsets, G + 1, "group_offsets")
    for t, n, name in ((X_perm, rows * H, "X_perm"), (W1_r, G * H * Fr, "W1_r"), (W2_r, G * Fr * H, "W2_r"),
                       (A1_r, rows * Fr, "A1_r"), (Y_r, rows * Fr, "Y_r"), (dZ_perm, rows * H, "dZ_perm"),
                       (dX_perm, rows * H, "dX_perm"), (dW1_r, G * H * Fr, "dW1_r"), (db1_r, G * Fr, "db1_r"),
                       (dW2_r, G * Fr * H, "dW2_r")):
        _need(t, n, name)
    dt = X_perm.dtype
    rc = raw().tp_mlp_grouped_shard_bwd(
        tp_size, rank, G, _ptr(group_offsets, "group_offsets", torch.int32), rows, H, F_group, _dtype_code(X_perm),
        _ptr(X_perm, "X_perm"), _ptr(W1_r, "W1_r", dt), _ptr(W2_r, "W2_r", dt), _ptr(A1_r, "A1_r", dt),
        _ptr(Y_r, "Y_r", dt), _ptr(dZ_perm, "dZ_perm", dt), _ptr(dX_perm, "dX_perm", dt), _ptr(dW1_r, "dW1_r", dt),
        _ptr(db1_r, "db1_r", dt), _ptr(dW2_r, "dW2_r", dt), _ptr(workspace, "workspace", None, True),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream))
    _check(rc, "tp_mlp_grouped_shard_bwd")


def tp_moe_shard_bwd(tp_size, rank, tokens, H, n_experts, top_k, F_expert, X, gates, group_offsets, row_token,
                     token_row, W1_r, W2_r, A1_r, Y_r, Z_r, d_out, dX_r, dgates_r, dW1_r, db1_r, dW2_r, workspace,
                     stream=None):
    """Backward of tp_moe_shard_fwd on this rank (partial dX_r and gate gradients; expert weight
    gradients of the rank's shards).  Z_r is not read (None is accepted)."""
    n = tokens * top_k
    _, Fr = tp_shard_range(F_expert, tp_size, rank) if 0 <= rank < tp_size and F_expert >= tp_size >= 1 else (0, 0)
    E = n_experts
    for t, m, name in ((X, tokens * H, "X"), (gates, n, "gates"), (group_offsets, E + 1, "group_offsets"),
                       (row_token, n, "row_token"), (token_row, n, "token_row"), (W1_r, E * H * Fr, "W1_r"),
                       (W2_r, E * Fr * H, "W2_r"), (A1_r, n * Fr, "A1_r"), (Y_r, n * Fr, "Y_r"), (d_out, tokens * H, "d_out"),
                       (dX_r, tokens * H, "dX_r"), (dgates_r, n, "dgates_r"), (dW1_r, E * H * Fr, "dW1_r"),
                       (db1_r, E * Fr, "db1_r"), (dW2_r, E * Fr * H, "dW2_r")):
        _need(t, m, name)
    dt = X.dtype
    rc = raw().tp_moe_shard_bwd(
        tp_size, rank, tokens, H, n_experts, top_k, F_expert, _dtype_code(X), _ptr(X, "X"),
        _ptr(gates, "gates", torch.float32), _ptr(group_offsets, "group_offsets", torch.int32),
        _ptr(row_token, "row_token", torch.int32), _ptr(token_row, "token_row", torch.int32),
        _ptr(W1_r, "W1_r", dt), _ptr(W2_r, "W2_r", dt),
        _ptr(A1_r, "A1_r", dt), _ptr(Y_r, "Y_r", dt), _ptr(Z_r, "Z_r", dt, True), _ptr(d_out, "d_out", dt),
        _ptr(dX_r, "dX_r", dt), _ptr(dgates_r, "dgates_r", torch.float32), _ptr(dW1_r, "dW1_r", dt),
        _ptr(db1_r, "db1_r", dt), _ptr(dW2_r, "dW2_r", dt), _ptr(workspace, "workspace", None, True),
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream(stream))
    _check(rc, "tp_moe_shard_bwd")


def tp_moe_route_bwd(logits, expert_idx, dgates, d_logits, stream=None):
    """Router logit gradient [tokens, E] from the gate gradient, the choice held fixed."""
    tokens, E = logits.shape
    k = expert_idx.shape[1]
    _need(dgates, tokens * k, "dgates")
    _need(d_logits, tokens * E, "d_logits")
    rc = raw().tp_moe_route_bwd(tokens, E, k, _ptr(logits, "logits", torch.float32),
                                _ptr(expert_idx, "expert_idx", torch.int32), _ptr(dgates, "dgates", torch.float32),
                                _ptr(d_logits, "d_logits", torch.float32), _stream(stream))
    _check(rc, "tp_moe_route_bwd")


def tp_bias_grad(dy, db, workspace, stream=None):
    """db [cols] = Σ over the rows of dy [rows, cols] (fixed-order fp32 sum, in dy's dtype)."""
    rows, cols = dy.shape
    _need(db, cols, "db")
    rc = raw().tp_bias_grad(rows, cols, _dtype_code(dy), _ptr(dy, "dy"), _ptr(db, "db", dy.dtype),
                            _ptr(workspace, "workspace", None, True),
                            workspace.numel() * workspace.element_size() if workspace is not None else 0,
                            _stream(stream))
    _check(rc, "tp_bias_grad")


def workspace(fn, tp_size, rank, B, S, H, n_heads, F, dtype, device="cuda"):
    """A caller-owned workspace tensor of the size the library asks for (None if it needs none)."""
    n = tp_workspace_bytes(fn, tp_size, rank, B, S, H, n_heads, F, dtype)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def tp_prof_enable(on: bool):
    _check(raw().tp_prof_enable(1 if on else 0), "tp_prof_enable")


def tp_prof_collect(max_entries=64, name_len=128):
    """Per-kernel-tag totals since the last collection: {tag: (launches, ms, flop, bytes)}."""
    names = ctypes.create_string_buffer(max_entries * name_len)
    n_l = (_I * max_entries)()
    ms, fl, by = ((ctypes.c_double * max_entries)() for _ in range(3))
    n = raw().tp_prof_collect(max_entries, names, name_len, n_l, ms, fl, by)
    if n < 0:
        raise TpError(n, "tp_prof_collect", raw().tp_last_error().decode())
    out = {}
    for i in range(min(n, max_entries)):
        tag = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[tag] = (n_l[i], ms[i], fl[i], by[i])
    return out
