"""Oracle for one rank's shard of multi-head self-attention (float64).

Heads are independent, so the Q, K and V weight matrices are split by columns
into blocks of whole heads, each rank runs attention on its own heads with no
communication, and the output projection is split by rows so that each rank
produces a partial of the layer output that the all-reduce adds
[Megatron-LM：张量并行与大规模训练, §2.2 Self-Attention 的张量并行; m.youleyou.com/
wenzhang/3143730, 三、Self-Attention层 §3.1].

Readings where the pages are silent or garbled:
  * per head: softmax(Q K^T / sqrt(d)) V with d_k = d_v = d = h / heads
    (the single-head formula itself is missing from the extract);
  * causal: key u is visible to query t iff u <= t (diagonal included);
  * a rank owns H/N contiguous heads; Wqkv_i columns are [Q | K | V] blocks of
    Hl*d columns each, head j at columns j*d .. (j+1)*d inside each block;
    Wo_i rows follow the same head order;
  * "matched" mode rounds Q, K, V and the concatenated head outputs O to
    bfloat16, where the GPU stores them. The softmax probabilities are not
    rounded here;
  * backward: the chain rule through the same formula, written out per head
    (dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = dS K / sqrt(d),
    dK = dS^T Q / sqrt(d)); the layer's two all-reduces (forward after Wo,
    backward of the input gradient) make the rank's dX_i a partial
    [m.youleyou.com/wenzhang/3143730, 三、Self-Attention层 §3.2]. Matched mode
    rounds dO = dOut Wo_i^T and dQKV to bfloat16, where the GPU stores them;
  * the row term rowsum(P * dP) equals rowsum(dO * O) with O = P V exactly. A
    training step keeps O only in its stored (bfloat16) form, so matched mode
    forms the term from the stored O, as the backward that consumes it does;
    the plain definition (no O given) forms rowsum(P * dP).
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


def _head_attention_bwd(q, k, v, do, causal, o=None):
    """Gradients of <do, softmax(q k^T / sqrt(d)) v> with respect to q, k, v.
    With o (the stored head output) the row term rowsum(P * dP) is taken as
    rowsum(do * o), its value when o = P v."""
    d = q.shape[1]
    S = (q @ k.T) / np.sqrt(d)
    if causal:
        t = np.arange(q.shape[0])[:, None]
        u = np.arange(k.shape[0])[None, :]
        S = np.where(u <= t, S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    dV = P.T @ do
    dP = do @ v.T
    rowterm = (P * dP).sum(axis=1, keepdims=True) if o is None else (do * o).sum(axis=1, keepdims=True)
    dS = P * (dP - rowterm)
    return dS @ k / np.sqrt(d), dS.T @ q / np.sqrt(d), dV


def attn_core_bwd(Q, K, V, dO, b, s, n_heads, d, causal=True, O=None):
    """Per-sequence, per-head attention backward. All [b*s, n_heads*d]. O (optional):
    the stored forward output, from which the row term rowsum(dO * O) is formed."""
    dQ, dK, dV = (np.empty_like(Q, dtype=np.float64) for _ in range(3))
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for j in range(n_heads):
            c = slice(j * d, (j + 1) * d)
            dQ[r, c], dK[r, c], dV[r, c] = _head_attention_bwd(Q[r, c], K[r, c], V[r, c], dO[r, c], causal,
                                                               None if O is None else O[r, c])
    return dQ, dK, dV


def attn_lse(Q, K, b, s, n_heads, d, causal=True):
    """log-sum-exp of each query's scaled scores, [b, n_heads, s] (natural log)."""
    out = np.empty((b, n_heads, s), np.float64)
    for bi in range(b):
        r = slice(bi * s, (bi + 1) * s)
        for j in range(n_heads):
            c = slice(j * d, (j + 1) * d)
            S = (Q[r, c] @ K[r, c].T) / np.sqrt(d)
            if causal:
                S = np.where(np.arange(s)[None, :] <= np.arange(s)[:, None], S, -np.inf)
            m = S.max(axis=1)
            out[bi, j] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return out


def attn_shard_bwd(X, Wqkv_i, Wo_i, dOut, b, s, n_heads_local, d, causal=True, matched=True):
    """One rank's attention backward: dWo_i = O^T dOut, dO = dOut Wo_i^T, the core
    backward, dWqkv_i = X^T dQKV and the input-gradient partial dX_i = dQKV Wqkv_i^T."""
    f = attn_shard(X, Wqkv_i, Wo_i, b, s, n_heads_local, d, causal, matched)
    dWo = f["O"].T @ dOut
    dO = _r(dOut @ Wo_i.T, matched)
    dQ, dK, dV = attn_core_bwd(f["Q"], f["K"], f["V"], dO, b, s, n_heads_local, d, causal,
                               O=f["O"] if matched else None)
    dQKV = _r(np.concatenate([dQ, dK, dV], axis=1), matched)
    return dict(fwd=f, dO=dO, dQKV=dQKV, dWo=dWo, dWqkv=X.T @ dQKV, dX=dQKV @ Wqkv_i.T)
