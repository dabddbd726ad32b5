"""Oracle for sequence parallelism around the MLP block of one layer.

Sequence parallelism [www.discosf.com/news/5875844, 2.3 序列并行与激活重计算]
takes the light operators that need the whole hidden row (LayerNorm, Dropout)
out of the per-rank replicated work: the sequence is cut into N contiguous row
ranges and rank i runs them on its own rows only. The MLP in between stays
tensor-parallel, so the all-reduce of its output is replaced by its two halves
[m.youleyou.com/wenzhang/3143730, 二、§2.2: an all-reduce is a reduce-scatter
followed by an all-gather, each moving the same volume]:

    R_i  [s/N, h]  rank i's rows of the residual stream (float32)
    L_i  = LayerNorm(R_i)                          (bf16 storage)
    X    = all_gather(L_0 .. L_{N-1})  [s, h]      every rank's input to f
    Z_j  = GeLU(X A_j) B_j             [s, h]      each rank's fp32 partial
    O_i  = reduce_scatter(Z_0 .. Z_{N-1})_i = sum_j Z_j[rows of i]
    R'_i = R_i + Dropout(O_i)

Readings (listed in the design doc):
  * LayerNorm is the standard one (not written out on the pages): per row, mean
    and biased variance over h, (x - mean) / sqrt(var + eps) * gamma + beta, with
    eps = 1e-5 and float32 gamma, beta [h];
  * Dropout's random draw is an input: a keep mask (1 keep, 0 drop) and the keep
    probability p; kept values are scaled by 1/p;
  * the residual stream stays float32; the LayerNorm output is stored bf16 (the
    GEMM's input dtype); the reduce-scatter adds the partials in rank order 0..N-1;
  * rank i owns rows [i*s/N, (i+1)*s/N).

float64 throughout; ``matched=True`` rounds the LayerNorm output to bf16 as the
GPU stores it.
"""
import numpy as np

from .bf16 import round_to_bf16
from .mlp import mlp_fwd_shard

LN_EPS = 1e-5


def layernorm(X, gamma, beta, eps=LN_EPS):
    """Row-wise LayerNorm: mean and biased variance over the last axis."""
    X = np.asarray(X, np.float64)
    mu = X.mean(axis=1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=1, keepdims=True)
    return (X - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def row_slice(s, N, i):
    """Rows [i*s/N, (i+1)*s/N) owned by rank i."""
    assert s % N == 0
    w = s // N
    return slice(i * w, (i + 1) * w)


def all_gather(slices):
    """Concatenate the ranks' row slices in rank order."""
    return np.concatenate([np.asarray(x) for x in slices], axis=0)


def reduce_scatter(partials, N, i):
    """Rank i's rows of the rank-ordered sum of the N partials."""
    rs = row_slice(partials[0].shape[0], N, i)
    out = np.zeros_like(np.asarray(partials[0][rs], np.float64))
    for P in partials:
        out = out + np.asarray(P[rs], np.float64)
    return out


def dropout_residual(R_i, O_i, keep=None, p=1.0):
    """R_i + Dropout(O_i): kept entries scaled by 1/p, dropped ones zero."""
    O = np.asarray(O_i, np.float64)
    if keep is not None:
        O = np.where(np.asarray(keep) != 0, O / p, 0.0)
    return np.asarray(R_i, np.float64) + O


def sp_mlp_block(R, gamma, beta, shards, keep=None, p=1.0, matched=True, eps=LN_EPS):
    """The whole sequence-parallel MLP block over N = len(shards) ranks.

    R [s, h] float32 residual rows; shards = [(A_j, B_j)]; keep [s, h] or None.
    Returns the per-rank intermediates and the new residual rows (all ranks)."""
    N = len(shards)
    s = R.shape[0]
    L = []
    for i in range(N):
        l_i = layernorm(R[row_slice(s, N, i)], gamma, beta, eps)
        L.append(round_to_bf16(l_i) if matched else l_i)
    X = all_gather(L)
    Z = [mlp_fwd_shard(X, A_j, B_j, matched=matched)["Z"] for A_j, B_j in shards]
    out = []
    for i in range(N):
        rs = row_slice(s, N, i)
        O_i = reduce_scatter(Z, N, i)
        out.append(dropout_residual(R[rs], O_i, None if keep is None else keep[rs], p))
    return dict(L=L, X=X, Z=Z, R_out=np.concatenate(out, axis=0))


def tp_mlp_block(R, gamma, beta, shards, keep=None, p=1.0, matched=True, eps=LN_EPS):
    """The same block without sequence parallelism: every rank runs LayerNorm on
    all s rows, the partials are all-reduced, and Dropout + residual run on all
    rows [Megatron-LM：张量并行与大规模训练, §2.1 (the MLP's single all-reduce)]."""
    X = layernorm(R, gamma, beta, eps)
    if matched:
        X = round_to_bf16(X)
    Z = None
    for A_j, B_j in shards:
        z = mlp_fwd_shard(X, A_j, B_j, matched=matched)["Z"]
        Z = z if Z is None else Z + z
    return dict(X=X, R_out=dropout_residual(R, Z, keep, p))
