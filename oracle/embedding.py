"""Oracle for the vocabulary-parallel input embedding of one rank.

The word-embedding table [v, h] is split by rows; a rank keeps the ids in its
range and looks them up, returns all-zero vectors for ids it does not hold,
and the all-reduce over ranks assembles the full lookup
[m.youleyou.com/wenzhang/3143730, 四、Embedding层 §4.1 输入层Embedding].

Reading: the range is half-open [lo, hi) (the page's two-way example of a
300-word vocabulary is read as [0, 150) and [150, 300)); ids outside [0, v)
hit no rank and give zero rows.

The lookup copies bit patterns; no arithmetic is involved.
"""
import numpy as np


def vocab_embed_shard(ids, E_i, lo, hi):
    """out[t] = E_i[ids[t] - lo] when lo <= ids[t] < hi, else a zero row.

    E_i holds rows lo .. hi-1 of the table (any dtype, e.g. bf16 bit patterns).
    """
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    E_i = np.asarray(E_i)
    assert E_i.shape[0] == hi - lo
    out = np.zeros((ids.shape[0],) + E_i.shape[1:], E_i.dtype)
    hit = (ids >= lo) & (ids < hi)
    out[hit] = E_i[ids[hit] - lo]
    return out
