"""Oracle for the tensor-parallel MLP shard, forward and backward (float64).

The MLP is Z = GeLU(X A) B with A [h, 4h] and B [4h, h]. Rank i of N holds the
column block A_i [h, 4h/N] and the row block B_i [4h/N, h]; it computes
Y_i = GeLU(X A_i) with no communication, because GeLU acts elementwise on the
columns it owns, then the partial Z_i = Y_i B_i; the all-reduce adds the Z_i
[Megatron-LM：张量并行与大规模训练, §2.1 MLP 层的张量并行, column and row parallelism and
the pseudo-code there; m.youleyou.com/wenzhang/3143730, 二、MLP层 §2.1].

Backward follows the conjugate operators of the same page's 一、切分权重 §1.1/§1.2 and
二、MLP层 §2.1: g's backward hands the replicated dZ to every rank unchanged, each
rank forms its own weight gradients and its input-gradient partial dX_i, and f's
backward adds the dX_i over ranks.

Readings where the pages are silent:
  * GeLU is the exact erf form x*Phi(x) (not the tanh approximation);
  * no bias, LayerNorm, residual or dropout inside the block;
  * "matched" mode rounds to bfloat16 exactly where the GPU stores bf16:
    U_i (saved pre-activation), Y_i, and dU_i. All other values stay float64.
"""
import numpy as np
from scipy.special import erf

from .bf16 import round_to_bf16

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def gelu(u):
    """GeLU(u) = u * Phi(u) = 0.5 * u * (1 + erf(u / sqrt 2))."""
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + erf(u / _SQRT2))


def gelu_prime(u):
    """d/du GeLU(u) = Phi(u) + u * phi(u), phi the standard normal density."""
    u = np.asarray(u, np.float64)
    return 0.5 * (1.0 + erf(u / _SQRT2)) + u * _INV_SQRT_2PI * np.exp(-0.5 * u * u)


def _r(x, matched):
    return round_to_bf16(x) if matched else x


def mlp_fwd_shard(X, A_i, B_i, matched=True):
    """One rank's forward: U_i = X A_i, Y_i = GeLU(U_i), Z_i = Y_i B_i.

    Inputs are float64 arrays holding the exact input values. Returns U_i and
    Y_i as stored (bf16-rounded in matched mode) and the float64 partial Z_i.
    """
    U = X @ A_i
    Y = _r(gelu(U), matched)
    U_s = _r(U, matched)
    Z = Y @ B_i
    return dict(U=U_s, Y=Y, Z=Z)


def mlp_bwd_shard(X, A_i, B_i, U_s, Y_s, dZ, matched=True):
    """One rank's backward given the replicated upstream gradient dZ.

    dY_i = dZ B_i^T;  dU_i = dY_i * GeLU'(U_i);  dB_i = Y_i^T dZ;
    dA_i = X^T dU_i;  dX_i = dU_i A_i^T (the partial that f's backward sums).
    U_s and Y_s are the stored forward activations (this oracle's own).
    """
    dY = dZ @ B_i.T
    dU = _r(dY * gelu_prime(U_s), matched)
    return dict(dU=dU, dB=Y_s.T @ dZ, dA=X.T @ dU, dX=dU @ A_i.T)


def mlp_fwd_full(X, A, B, matched=False):
    """Unsharded Z = GeLU(X A) B in float64 (the all-reduced result). With
    matched=True the activation is rounded to bf16 before the second product,
    exactly as each rank stores its own column block of it."""
    return _r(gelu(X @ A), matched) @ B


def mlp_bwd_full(X, A, B, dZ):
    """Unsharded gradients of L = <dZ, GeLU(X A) B> in float64: (dX, dA, dB)."""
    U = X @ A
    dU = (dZ @ B.T) * gelu_prime(U)
    return dict(dX=dU @ A.T, dA=X.T @ dU, dB=gelu(U).T @ dZ)


def mlp_fwd_rows(X, A_i, B_i, rows, matched=True):
    """mlp_fwd_shard restricted to the token rows `rows` (rows are independent)."""
    out = mlp_fwd_shard(X[rows], A_i, B_i, matched)
    return out


def mlp_bwd_cols(X, A_i, B_i, dZ, rows, cols, matched=True):
    """Sampled backward outputs of one rank, each computed from its definition.

    Returns dU[:, cols], dA[:, cols], dB[cols, :] (these need every token of the
    chosen hidden columns q of the shard) and dX[rows, :] (needs every column
    of the chosen token rows). The forward activations U, Y are recomputed here
    for exactly the entries needed, with the same storage rounding.
    """
    # columns q of U, Y over all tokens
    Uc = X @ A_i[:, cols]
    Uc_s = _r(Uc, matched)
    Yc_s = _r(gelu(Uc), matched)
    dU_c = _r((dZ @ B_i[cols, :].T) * gelu_prime(Uc_s), matched)
    dA_c = X.T @ dU_c
    dB_r = Yc_s.T @ dZ
    # rows t of dU over all columns, then dX rows
    Ur = X[rows] @ A_i
    dU_r = _r((dZ[rows] @ B_i.T) * gelu_prime(_r(Ur, matched)), matched)
    dX_r = dU_r @ A_i.T
    return dict(dU_cols=dU_c, dA_cols=dA_c, dB_rows=dB_r, dX_rows=dX_r, dU_rows=dU_r)
