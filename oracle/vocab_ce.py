"""Oracle for the vocabulary-parallel output layer and its cross-entropy loss.

The output layer maps each hidden row back to the vocabulary with the (shared)
word-embedding table, split by rows over the ranks, so rank i produces the
logits of its own vocabulary slice [lo, hi): logits_i = H E_i^T
[m.youleyou.com/wenzhang/3143730, 四、Embedding层 §4.2 输出层Embedding].

The loss avoids gathering the logits: every rank sums e = exp(logit) over its
own columns, row by row; an all-reduce of those sums gives the softmax
denominator sum(e) of every row; the rank that holds a row's target turns its
e / sum(e) into that row's cross-entropy; the rows' losses are added into a
scalar, and a last all-reduce adds the ranks' scalars
[same page, 五、Cross-Entropy层].

Readings:
  * e is exp(logit) itself, as the page states it: no row maximum is subtracted
    (float32 logits above about 88 would overflow; the workloads stay far below);
  * a row's loss is -log(e_t / sum(e)) = log(sum(e)) - logit_t for its target t;
  * the scalar loss is the plain sum over rows (the page says the rows' losses
    are summed);
  * the vocabulary slice of rank i is [lo, hi), as for the input embedding;
  * the rank-local results are (sumexp_i, tlogit_i) per row, tlogit_i being the
    target's logit when the target is in [lo, hi) and 0 otherwise; the two
    all-reduce stand-ins add them over the ranks in the fixed order 0..N-1.

float64 throughout; inputs are the bf16-stored H and E_i as float64.
"""
import numpy as np


def vocab_ce_partials(H, E_i, targets, lo, hi):
    """One rank's part: logits_i = H E_i^T, and per row the sum of exp over the
    rank's columns and the target's logit when the rank holds the target (else 0)."""
    H = np.asarray(H, np.float64)
    E_i = np.asarray(E_i, np.float64)
    t = np.asarray(targets, np.int64).reshape(-1)
    assert E_i.shape[0] == hi - lo and H.shape[1] == E_i.shape[1] and t.shape[0] == H.shape[0]
    logits = H @ E_i.T
    sumexp = np.exp(logits).sum(axis=1)
    hit = (t >= lo) & (t < hi)
    tlogit = np.zeros(H.shape[0], np.float64)
    tlogit[hit] = logits[np.nonzero(hit)[0], t[hit] - lo]
    return dict(logits=logits, sumexp=sumexp, tlogit=tlogit)


def vocab_ce_combine(sumexp_parts, tlogit_parts):
    """The all-reduce stand-ins and the loss: S = sum_i sumexp_i, loss_row =
    log(S) - sum_i tlogit_i, loss = sum of the rows."""
    S = np.zeros_like(np.asarray(sumexp_parts[0], np.float64))
    T = np.zeros_like(S)
    for s_i, t_i in zip(sumexp_parts, tlogit_parts):
        S = S + np.asarray(s_i, np.float64)
        T = T + np.asarray(t_i, np.float64)
    rows = np.log(S) - T
    return dict(sumexp=S, loss_rows=rows, loss=float(rows.sum()))


def vocab_ce_sharded(H, E, targets, N):
    """Whole vocabulary-parallel loss over N equal row slices of E [v, h]."""
    v = E.shape[0]
    parts = [vocab_ce_partials(H, E[i * v // N:(i + 1) * v // N], targets, i * v // N, (i + 1) * v // N)
             for i in range(N)]
    return vocab_ce_combine([p["sumexp"] for p in parts], [p["tlogit"] for p in parts])
