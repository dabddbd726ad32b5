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

Readings:
  * LayerNorm is the standard one (not written out on the pages): per row, mean
    and biased variance over h, (x - mean) / sqrt(var + eps) * gamma + beta, with
    eps = 1e-5 and float32 gamma, beta [h];
  * Dropout's random draw is an input: a keep mask (1 keep, 0 drop) and the keep
    probability p; kept values are scaled by 1/p;
  * the residual stream stays float32; the LayerNorm output is stored bf16 (the
    GEMM's input dtype); the reduce-scatter adds the partials in rank order 0..N-1;
  * rank i owns rows [i*s/N, (i+1)*s/N).

Backward (the chain rule through the same block; the page states only the
forward split): Dropout's backward scales the kept gradient by 1/p; the
reduce-scatter's backward is an all-gather of the ranks' gradient rows (the
MLP's replicated upstream gradient); the all-gather's backward is a
reduce-scatter of the MLP's input-gradient partials; LayerNorm's backward runs
on the rank's rows, and its gamma, beta gradients are per-rank partials that an
all-reduce adds. The residual path passes the gradient through.

float64 throughout; ``matched=True`` rounds the LayerNorm output, and in the
backward the gathered upstream gradient, to bf16 as the GPU stores them.
"""
import numpy as np

from .bf16 import round_to_bf16
from .mlp import mlp_bwd_shard, mlp_fwd_shard

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


def layernorm_bwd(X, gamma, dY, eps=LN_EPS):
    """Gradients of sum(dY * LayerNorm(X)) with respect to X, gamma and beta.

    With xh = (x - mean) * rstd and g = dY * gamma, per row:
    dX = rstd * (g - mean(g) - xh * mean(g * xh)); dgamma = sum_rows dY * xh;
    dbeta = sum_rows dY."""
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    mu = X.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((X - mu) ** 2).mean(axis=1, keepdims=True) + eps)
    xh = (X - mu) * rstd
    g = dY * np.asarray(gamma, np.float64)
    dX = rstd * (g - g.mean(axis=1, keepdims=True) - xh * (g * xh).mean(axis=1, keepdims=True))
    return dict(dX=dX, dgamma=(dY * xh).sum(axis=0), dbeta=dY.sum(axis=0))


def dropout_bwd(dY, keep=None, p=1.0):
    """Gradient through Dropout: kept entries scaled by 1/p, dropped ones zero."""
    dY = np.asarray(dY, np.float64)
    if keep is None:
        return dY
    return np.where(np.asarray(keep) != 0, dY / p, 0.0)


def sp_mlp_block_bwd(R, gamma, beta, shards, dR_out, keep=None, p=1.0, matched=True, eps=LN_EPS):
    """Backward of sp_mlp_block for the upstream gradient dR_out [s, h] of the new
    residual rows. Returns dR (all ranks' rows), dgamma and dbeta (summed over the
    ranks' partials), the per-rank partials, and each rank's dA_j, dB_j."""
    N = len(shards)
    s = R.shape[0]
    f = sp_mlp_block(R, gamma, beta, shards, keep, p, matched, eps)
    fw = [mlp_fwd_shard(f["X"], A_j, B_j, matched=matched) for A_j, B_j in shards]
    dO = [dropout_bwd(dR_out[row_slice(s, N, i)], None if keep is None else keep[row_slice(s, N, i)], p)
          for i in range(N)]
    dZ = all_gather(dO)
    if matched:
        dZ = round_to_bf16(dZ)
    g = [mlp_bwd_shard(f["X"], A_j, B_j, fw[j]["U"], fw[j]["Y"], dZ, matched=matched)
         for j, (A_j, B_j) in enumerate(shards)]
    dX_parts = [gj["dX"] for gj in g]
    dR, dgam, dbet = [], [], []
    for i in range(N):
        rs = row_slice(s, N, i)
        dL_i = reduce_scatter(dX_parts, N, i)
        lb = layernorm_bwd(R[rs], gamma, dL_i, eps)
        dR.append(np.asarray(dR_out[rs], np.float64) + lb["dX"])
        dgam.append(lb["dgamma"])
        dbet.append(lb["dbeta"])
    return dict(dR=np.concatenate(dR, axis=0), dgamma=sum(dgam), dbeta=sum(dbet), dgamma_parts=dgam,
                dbeta_parts=dbet, dZ=dZ, dX_parts=dX_parts, dA=[gj["dA"] for gj in g], dB=[gj["dB"] for gj in g])
