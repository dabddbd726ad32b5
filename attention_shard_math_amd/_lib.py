"""ctypes binding of the libtpshard C ABI (include/tpshard.h).

Each function takes torch tensors, checks dtype/shape/contiguity/device (the C
side cannot see tensor metadata), passes raw device pointers plus the current
HIP stream, and raises TpError on a non-OK status.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python attention_shard_math_amd/build.py` "
                      "(or __graft_entry__.build()) first")
lib = C.CDLL(LIB_PATH)

TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU = 0, 1
_i64, _vp, _sz = C.c_int64, C.c_void_p, C.c_size_t

_SIGS = {
    "tp_column_linear": [C.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, C.c_int, _vp, _sz, _vp],
    "tp_row_linear": [C.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_mlp_fwd": [C.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_mlp_bwd": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_mlp_bwd_noalloc": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_attn_core": [_i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp],
    "tp_attn_fwd": [_i64, _i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_vocab_embed": [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _vp],
    "tp_shard_sum": [C.c_int, C.POINTER(_vp), C.c_int, _i64, _vp, _vp],
    "tp_vocab_ce_partials": [_i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_vocab_ce_loss": [_i64, C.POINTER(_vp), C.POINTER(_vp), C.POINTER(_vp), C.c_int, _vp, _vp, _vp],
    "tp_attn_core_train": [_i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp],
    "tp_attn_fwd_train": [_i64, _i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "tp_attn_core_bwd": [_i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_attn_bwd": [_i64, _i64, _i64, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                    _sz, _vp],
    "tp_layernorm": [_i64, _i64, _vp, _vp, _vp, C.c_float, _vp, _vp],
    "tp_sp_all_gather": [C.c_int, C.POINTER(_vp), _i64, _i64, _vp, _vp],
    "tp_layernorm_bwd": [_i64, _i64, _vp, _vp, _vp, _vp, C.c_float, _vp, _vp, _vp, _vp, _sz, _vp],
    "tp_sp_dropout_bwd": [_i64, _i64, _vp, _vp, C.c_float, _vp, _vp],
    "tp_sp_reduce_scatter": [C.c_int, C.POINTER(_vp), _i64, _i64, C.c_int, _vp, _vp, C.c_float, _vp, _vp],
}
for _name, _args in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = C.c_int
lib.tp_mlp_bwd_workspace.argtypes = [_i64, _i64, _i64]
lib.tp_mlp_bwd_workspace.restype = _sz
lib.tp_mlp_bwd_recompute_workspace.argtypes = [_i64, _i64, _i64]
lib.tp_mlp_bwd_recompute_workspace.restype = _sz
lib.tp_vocab_ce_workspace.argtypes = [_i64, _i64, _i64, _i64]
lib.tp_layernorm_bwd_workspace.argtypes = [_i64, _i64]
lib.tp_layernorm_bwd_workspace.restype = _sz
lib.tp_attn_core_bwd_workspace.argtypes = [_i64, _i64, _i64, _i64]
lib.tp_attn_core_bwd_workspace.restype = _sz
lib.tp_attn_bwd_workspace.argtypes = [_i64, _i64, _i64, _i64, _i64]
lib.tp_attn_bwd_workspace.restype = _sz
lib.tp_vocab_ce_workspace.restype = _sz
lib.tp_attn_fwd_workspace.argtypes = [_i64, _i64, _i64, _i64, _i64]
lib.tp_attn_fwd_workspace.restype = _sz
lib.tp_linear_workspace.argtypes = [C.c_int, _i64, _i64, _i64]
lib.tp_linear_workspace.restype = _sz
lib.tp_mlp_fwd_workspace.argtypes = [C.c_int, _i64, _i64, _i64]
lib.tp_mlp_fwd_workspace.restype = _sz
lib.tp_mlp_bwd_noalloc_max_bytes.argtypes = []
lib.tp_mlp_bwd_noalloc_max_bytes.restype = _sz
lib.tp_status_string.argtypes = [C.c_int]
lib.tp_status_string.restype = C.c_char_p
lib.tp_last_error.argtypes = []
lib.tp_last_error.restype = C.c_char_p


class TpError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        msg = lib.tp_last_error().decode()
        super().__init__(f"{fn}: {lib.tp_status_string(status).decode()}: {msg}")


def _check(status: int, fn: str):
    if status != 0:
        raise TpError(status, fn)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TP_F32
    if t.dtype == torch.bfloat16:
        return TP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, shape=None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _wsargs(ws):
    return (None, 0) if ws is None else (_ptr(ws, name="ws"), ws.numel() * ws.element_size())


def linear_workspace(M, K, N, dtype=torch.bfloat16) -> int:
    return int(lib.tp_linear_workspace(TP_BF16 if dtype == torch.bfloat16 else TP_F32, M, K, N))


def column_linear(X, W, Y, U=None, act="gelu", ws=None, stream=None):
    """Y = act(X W) (and U = X W when act is GeLU and U is given)."""
    M, K = X.shape
    N = W.shape[1]
    dt = X.dtype
    a = TP_ACT_GELU if act == "gelu" else TP_ACT_NONE
    wp, wb = _wsargs(ws)
    _check(lib.tp_column_linear(_dt(X), M, K, N, _ptr(X, (M, K), dt, "X"), _ptr(W, (K, N), dt, "W"),
                                _ptr(U, (M, N), dt, "U"), _ptr(Y, (M, N), dt, "Y"), a, wp, wb, _stream(stream)),
           "tp_column_linear")


def row_linear(Y, W, Z, ws=None, stream=None):
    """Z (float32) = Y W."""
    M, K = Y.shape
    N = W.shape[1]
    dt = Y.dtype
    wp, wb = _wsargs(ws)
    _check(lib.tp_row_linear(_dt(Y), M, K, N, _ptr(Y, (M, K), dt, "Y"), _ptr(W, (K, N), dt, "W"),
                             _ptr(Z, (M, N), torch.float32, "Z"), wp, wb, _stream(stream)), "tp_row_linear")


def mlp_fwd_workspace(M, h, f, dtype=torch.bfloat16) -> int:
    return int(lib.tp_mlp_fwd_workspace(TP_BF16 if dtype == torch.bfloat16 else TP_F32, M, h, f))


def mlp_fwd(X, A_i, B_i, Y_i, Z_i, U_i=None, ws=None, stream=None):
    M, h = X.shape
    f = A_i.shape[1]
    dt = X.dtype
    wp, wb = _wsargs(ws)
    _check(lib.tp_mlp_fwd(_dt(X), M, h, f, _ptr(X, (M, h), dt, "X"), _ptr(A_i, (h, f), dt, "A_i"),
                          _ptr(B_i, (f, h), dt, "B_i"), _ptr(U_i, (M, f), dt, "U_i"), _ptr(Y_i, (M, f), dt, "Y_i"),
                          _ptr(Z_i, (M, h), torch.float32, "Z_i"), wp, wb, _stream(stream)), "tp_mlp_fwd")


def mlp_bwd_workspace(M, h, f) -> int:
    return int(lib.tp_mlp_bwd_workspace(M, h, f))


def mlp_bwd_recompute_workspace(M, h, f) -> int:
    return int(lib.tp_mlp_bwd_recompute_workspace(M, h, f))


def mlp_bwd(X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i, ws, stream=None):
    M, h = X.shape
    f = A_i.shape[1]
    bf = torch.bfloat16
    f32 = torch.float32
    wsp = _ptr(ws, name="ws") if ws is not None else None
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib.tp_mlp_bwd(M, h, f, _ptr(X, (M, h), bf, "X"), _ptr(A_i, (h, f), bf, "A_i"),
                          _ptr(B_i, (f, h), bf, "B_i"), _ptr(U_i, (M, f), bf, "U_i"), _ptr(Y_i, (M, f), bf, "Y_i"),
                          _ptr(dZ, (M, h), bf, "dZ"), _ptr(dX_i, (M, h), f32, "dX_i"),
                          _ptr(dA_i, (h, f), f32, "dA_i"), _ptr(dB_i, (f, h), f32, "dB_i"), wsp, wsb,
                          _stream(stream)), "tp_mlp_bwd")


def attn_core(QKV, O, b, s, n_heads_local, d_head, causal=True, stream=None):
    w = n_heads_local * d_head
    bf = torch.bfloat16
    _check(lib.tp_attn_core(b, s, n_heads_local, d_head, int(causal), _ptr(QKV, (b * s, 3 * w), bf, "QKV"),
                            _ptr(O, (b * s, w), bf, "O"), _stream(stream)), "tp_attn_core")


def attn_fwd_workspace(b, s, n_heads_local, d_head, h) -> int:
    return int(lib.tp_attn_fwd_workspace(b, s, h, n_heads_local, d_head))


def attn_fwd(X, Wqkv_i, Wo_i, out, ws, b, s, n_heads_local, d_head, causal=True, stream=None):
    h = X.shape[1]
    w = n_heads_local * d_head
    bf = torch.bfloat16
    wsp = _ptr(ws, name="ws") if ws is not None else None
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib.tp_attn_fwd(b, s, h, n_heads_local, d_head, int(causal), _ptr(X, (b * s, h), bf, "X"),
                           _ptr(Wqkv_i, (h, 3 * w), bf, "Wqkv_i"), _ptr(Wo_i, (w, h), bf, "Wo_i"),
                           _ptr(out, (b * s, h), torch.float32, "out"), wsp, wsb, _stream(stream)), "tp_attn_fwd")


def vocab_embed(ids, E_i, lo, hi, out, stream=None):
    n = ids.numel()
    h = E_i.shape[1]
    bf = torch.bfloat16
    _check(lib.tp_vocab_embed(_ptr(ids, dtype=torch.int32, name="ids"), n, _ptr(E_i, (hi - lo, h), bf, "E_i"),
                              lo, hi, h, _ptr(out, (n, h), bf, "out"), _stream(stream)), "tp_vocab_embed")


def attn_core_train(QKV, O, lse, b, s, n_heads_local, d_head, causal=True, stream=None):
    w = n_heads_local * d_head
    bf = torch.bfloat16
    _check(lib.tp_attn_core_train(b, s, n_heads_local, d_head, int(causal), _ptr(QKV, (b * s, 3 * w), bf, "QKV"),
                                  _ptr(O, (b * s, w), bf, "O"), _ptr(lse, (b, n_heads_local, s), torch.float32, "lse"),
                                  _stream(stream)), "tp_attn_core_train")


def attn_fwd_train(X, Wqkv_i, Wo_i, out_partial, QKV, O, lse, b, s, n_heads_local, d_head, causal=True,
                   stream=None):
    h = X.shape[1]
    w = n_heads_local * d_head
    bf = torch.bfloat16
    _check(lib.tp_attn_fwd_train(b, s, h, n_heads_local, d_head, int(causal), _ptr(X, (b * s, h), bf, "X"),
                                 _ptr(Wqkv_i, (h, 3 * w), bf, "Wqkv_i"), _ptr(Wo_i, (w, h), bf, "Wo_i"),
                                 _ptr(out_partial, (b * s, h), torch.float32, "out_partial"),
                                 _ptr(QKV, (b * s, 3 * w), bf, "QKV"), _ptr(O, (b * s, w), bf, "O"),
                                 _ptr(lse, (b, n_heads_local, s), torch.float32, "lse"), _stream(stream)),
           "tp_attn_fwd_train")


def attn_core_bwd_workspace(b, s, n_heads_local, d_head):
    return int(lib.tp_attn_core_bwd_workspace(b, s, n_heads_local, d_head))


def attn_core_bwd(QKV, O, dO, lse, dQKV, ws, b, s, n_heads_local, d_head, causal=True, stream=None):
    w = n_heads_local * d_head
    bf = torch.bfloat16
    wp, wb = _wsargs(ws)
    _check(lib.tp_attn_core_bwd(b, s, n_heads_local, d_head, int(causal), _ptr(QKV, (b * s, 3 * w), bf, "QKV"),
                                _ptr(O, (b * s, w), bf, "O"), _ptr(dO, (b * s, w), bf, "dO"),
                                _ptr(lse, (b, n_heads_local, s), torch.float32, "lse"),
                                _ptr(dQKV, (b * s, 3 * w), bf, "dQKV"), wp, wb, _stream(stream)), "tp_attn_core_bwd")


def attn_bwd_workspace(b, s, h, n_heads_local, d_head):
    return int(lib.tp_attn_bwd_workspace(b, s, h, n_heads_local, d_head))


def attn_bwd(X, Wqkv_i, Wo_i, QKV, O, lse, dOut, dX_i, dWqkv_i, dWo_i, ws, b, s, n_heads_local, d_head,
             causal=True, stream=None):
    h = X.shape[1]
    w = n_heads_local * d_head
    bf, f32 = torch.bfloat16, torch.float32
    wp, wb = _wsargs(ws)
    _check(lib.tp_attn_bwd(b, s, h, n_heads_local, d_head, int(causal), _ptr(X, (b * s, h), bf, "X"),
                           _ptr(Wqkv_i, (h, 3 * w), bf, "Wqkv_i"), _ptr(Wo_i, (w, h), bf, "Wo_i"),
                           _ptr(QKV, (b * s, 3 * w), bf, "QKV"), _ptr(O, (b * s, w), bf, "O"),
                           _ptr(lse, (b, n_heads_local, s), f32, "lse"), _ptr(dOut, (b * s, h), bf, "dOut"),
                           _ptr(dX_i, (b * s, h), f32, "dX_i"), _ptr(dWqkv_i, (h, 3 * w), f32, "dWqkv_i"),
                           _ptr(dWo_i, (w, h), f32, "dWo_i"), wp, wb, _stream(stream)), "tp_attn_bwd")


def vocab_ce_workspace(M, h, lo, hi):
    return int(lib.tp_vocab_ce_workspace(M, h, lo, hi))


def vocab_ce_partials(H, E_i, targets, lo, hi, rowmax_i, sumexp_i, tlogit_i, ws, stream=None):
    M, h = H.shape
    V = hi - lo
    f32 = torch.float32
    _check(lib.tp_vocab_ce_partials(M, h, lo, hi, _ptr(H, (M, h), torch.bfloat16, "H"),
                                    _ptr(E_i, (V, h), torch.bfloat16, "E_i"),
                                    _ptr(targets, (M,), torch.int32, "targets"),
                                    _ptr(rowmax_i, (M,), f32, "rowmax_i"),
                                    _ptr(sumexp_i, (M,), f32, "sumexp_i"),
                                    _ptr(tlogit_i, (M,), f32, "tlogit_i"),
                                    *_wsargs(ws), _stream(stream)), "tp_vocab_ce_partials")


def vocab_ce_loss(rowmax_parts, sumexp_parts, tlogit_parts, loss_rows, loss_sum, stream=None):
    n = len(sumexp_parts)
    if len(tlogit_parts) != n or len(rowmax_parts) != n:
        raise ValueError("rowmax_parts, sumexp_parts and tlogit_parts differ in length")
    M = loss_rows.numel()

    def arr(parts, name):
        return (_vp * max(n, 1))(*[_ptr(p, (M,), torch.float32, f"{name}[{i}]") for i, p in enumerate(parts)])

    _check(lib.tp_vocab_ce_loss(M, arr(rowmax_parts, "rowmax_parts"), arr(sumexp_parts, "sumexp_parts"),
                                arr(tlogit_parts, "tlogit_parts"), n,
                                _ptr(loss_rows, (M,), torch.float32, "loss_rows"),
                                _ptr(loss_sum, (1,), torch.float32, "loss_sum"), _stream(stream)),
           "tp_vocab_ce_loss")


def layernorm(X, gamma, beta, Y, eps=1e-5, stream=None):
    """Y (bf16) = LayerNorm(X) row by row; X float32 [rows, h]."""
    rows, h = X.shape
    f32 = torch.float32
    _check(lib.tp_layernorm(rows, h, _ptr(X, (rows, h), f32, "X"), _ptr(gamma, (h,), f32, "gamma"),
                            _ptr(beta, (h,), f32, "beta"), eps, _ptr(Y, (rows, h), torch.bfloat16, "Y"),
                            _stream(stream)), "tp_layernorm")


def layernorm_bwd_workspace(rows, h):
    return int(lib.tp_layernorm_bwd_workspace(rows, h))


def layernorm_bwd(X, gamma, dY, dX, dgamma, dbeta, ws, dRes=None, eps=1e-5, stream=None):
    rows, h = X.shape
    f32 = torch.float32
    wp, wb = _wsargs(ws)
    _check(lib.tp_layernorm_bwd(rows, h, _ptr(X, (rows, h), f32, "X"), _ptr(gamma, (h,), f32, "gamma"),
                                _ptr(dY, (rows, h), f32, "dY"), _ptr(dRes, (rows, h), f32, "dRes"), eps,
                                _ptr(dX, (rows, h), f32, "dX"), _ptr(dgamma, (h,), f32, "dgamma"),
                                _ptr(dbeta, (h,), f32, "dbeta"), wp, wb, _stream(stream)), "tp_layernorm_bwd")


def sp_dropout_bwd(dY, out, keep=None, keep_prob=1.0, stream=None):
    rows, h = dY.shape
    _check(lib.tp_sp_dropout_bwd(rows, h, _ptr(dY, (rows, h), torch.float32, "dY"),
                                 _ptr(keep, (rows, h), torch.uint8, "keep"), keep_prob,
                                 _ptr(out, (rows, h), torch.bfloat16, "out"), _stream(stream)), "tp_sp_dropout_bwd")


def sp_all_gather(slices, out, stream=None):
    n = len(slices)
    rows, h = slices[0].shape
    arr = (_vp * max(n, 1))(*[_ptr(x, (rows, h), torch.bfloat16, f"slices[{i}]") for i, x in enumerate(slices)])
    _check(lib.tp_sp_all_gather(n, arr, rows, h, _ptr(out, (n * rows, h), torch.bfloat16, "out"), _stream(stream)),
           "tp_sp_all_gather")


def sp_reduce_scatter(partials, rank, residual, out, keep=None, keep_prob=1.0, stream=None):
    n = len(partials)
    s, h = partials[0].shape
    f32 = torch.float32
    arr = (_vp * max(n, 1))(*[_ptr(p, (s, h), f32, f"partials[{i}]") for i, p in enumerate(partials)])
    rows = s // n
    _check(lib.tp_sp_reduce_scatter(n, arr, s, h, rank, _ptr(residual, (rows, h), f32, "residual"),
                                    _ptr(keep, (rows, h), torch.uint8, "keep"), keep_prob,
                                    _ptr(out, (rows, h), f32, "out"), _stream(stream)), "tp_sp_reduce_scatter")


def shard_sum(partials, out, stream=None):
    n = len(partials)
    numel = out.numel()
    arr = (_vp * max(n, 1))(*[_ptr(p, dtype=out.dtype, name=f"partials[{i}]") for i, p in enumerate(partials)])
    for i, p in enumerate(partials):
        if p.numel() != numel:
            raise ValueError(f"partials[{i}] has {p.numel()} elements, out has {numel}")
    _check(lib.tp_shard_sum(_dt(out), arr, n, numel, _ptr(out, name="out"), _stream(stream)), "tp_shard_sum")


def mlp_bwd_noalloc_max_bytes() -> int:
    return int(lib.tp_mlp_bwd_noalloc_max_bytes())


def mlp_bwd_noalloc(X, A_i, B_i, U_i, Y_i, dZ, dX_i, dA_i, dB_i, stream=None):
    """tp_mlp_bwd without a workspace: dU lives in the library's per-device scratch."""
    M, h = X.shape
    f = A_i.shape[1]
    bf, f32 = torch.bfloat16, torch.float32
    _check(lib.tp_mlp_bwd_noalloc(M, h, f, _ptr(X, (M, h), bf, "X"), _ptr(A_i, (h, f), bf, "A_i"),
                                  _ptr(B_i, (f, h), bf, "B_i"), _ptr(U_i, (M, f), bf, "U_i"),
                                  _ptr(Y_i, (M, f), bf, "Y_i"), _ptr(dZ, (M, h), bf, "dZ"),
                                  _ptr(dX_i, (M, h), f32, "dX_i"), _ptr(dA_i, (h, f), f32, "dA_i"),
                                  _ptr(dB_i, (f, h), f32, "dB_i"), _stream(stream)), "tp_mlp_bwd_noalloc")
