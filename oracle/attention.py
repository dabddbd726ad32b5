"""Oracle for one rank's shard of multi-head self-attention (float64).

Heads are independent, so the Q, K and V weight matrices are split by columns
into blocks of whole heads, each rank runs attention on its own heads with no
communication, and the output projection is split by rows so that each rank
produces a partial of the layer output that the all-reduce adds
[Megatron-LM：张量并行与大规模训练, §2.2 Self-Attention 的张量并行; m.youleyou.com/
wenzhang/3143730, 三、Self-Attention层 §3.1].

Readings where the pages are silent or garbled (listed in the design doc):
  * per head: softmax(Q K^T / sqrt(d)) V with d_k = d_v = d = h / heads
    (the single-head formula itself is missing from the extract);
  * causal: key u is visible to query t iff u <= t (diagonal included);
  * a rank owns H/N contiguous heads; Wqkv_i columns are [Q | K | V] blocks of
    Hl*d columns each, head j at columns j*d .. (j+1)*d inside each block;
    Wo_i rows follow the same head order;
  * "matched" mode rounds Q, K, V and the concatenated head outputs O to
    bfloat16, where the GPU stores them. The softmax probabilities are not
    rounded here.
"""
import numpy as np

from .bf16 import round_to_bf16


def _r(x, matched):
    return round_to_bf16(x) if matched else x


def _head_attention(q, k, v, causal):
    """softmax(q k^T / sqrt(d)) v for one head of one sequence."""
    d = q.shape[1]
    S = (q @ k.T) / np.sqrt(d)
    if causal:
        t = np.arange(q.shape[0])[:, None]
        u = np.arange(k.shape[0])[None, :]
        S = np.where(u <= t, S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    return P @ v


def attn_core(Q, K, V, b, s, n_heads, d, causal=True):
    """Per-sequence, per-head attention. Q, K, V: [b*s, n_heads*d] -> O same shape."""
    O = np.empty_like(Q, dtype=np.float64)
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for j in range(n_heads):
            c = slice(j * d, (j + 1) * d)
            O[r, c] = _head_attention(Q[r, c], K[r, c], V[r, c], causal)
    return O


def _split_qkv(QKV, n_heads, d):
    w = n_heads * d
    return QKV[:, :w], QKV[:, w:2 * w], QKV[:, 2 * w:3 * w]


def attn_shard(X, Wqkv_i, Wo_i, b, s, n_heads_local, d, causal=True, matched=True):
    """One rank: [Q|K|V] = X Wqkv_i; O = attention over its local heads;
    out_i = O Wo_i (the partial that the all-reduce adds)."""
    Q, K, V = (_r(t, matched) for t in _split_qkv(X @ Wqkv_i, n_heads_local, d))
    O = _r(attn_core(Q, K, V, b, s, n_heads_local, d, causal), matched)
    return dict(Q=Q, K=K, V=V, O=O, out=O @ Wo_i)


def mha_full(X, Wq, Wk, Wv, Wo, b, s, n_heads, d, causal=True):
    """Unsharded multi-head attention output (float64, no storage rounding)."""
    O = attn_core(X @ Wq, X @ Wk, X @ Wv, b, s, n_heads, d, causal)
    return O @ Wo


def attn_shard_rows(X, Wqkv_i, Wo_i, b, s, n_heads_local, d, rows, causal=True,
                    matched=True):
    """attn_shard's output restricted to token rows `rows` (global indices in
    [0, b*s)). K and V are formed for every token; Q only for the chosen rows."""
    w = n_heads_local * d
    K = _r(X @ Wqkv_i[:, w:2 * w], matched)
    V = _r(X @ Wqkv_i[:, 2 * w:3 * w], matched)
    rows = np.asarray(rows)
    Q = _r(X[rows] @ Wqkv_i[:, :w], matched)
    O = np.empty((rows.shape[0], w), np.float64)
    for n, t in enumerate(rows):
        bi, p = divmod(int(t), s)
        last = p + 1 if causal else s
        kr = slice(bi * s, bi * s + last)
        for j in range(n_heads_local):
            c = slice(j * d, (j + 1) * d)
            sc = (K[kr, c] @ Q[n, c]) / np.sqrt(d)
            e = np.exp(sc - sc.max())
            O[n, c] = (e / e.sum()) @ V[kr, c]
    O = _r(O, matched)
    return dict(O=O, out=O @ Wo_i)
