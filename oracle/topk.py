"""Top-k selection of compressed entries (test infrastructure).

Pages: the indexer keeps the k compressed entries most relevant to the query
and attention runs only over those (blog.nickys.cn DeepSeek-V4 post,
三大架构改动 §1 CSA; sz-guanghua.com.cn ifanr repost, 百萬長上下文 section).

Readings where the pages are silent:
  * candidates are the visible entries e < nvis(t) = floor((t+1)/m);
  * order by score descending, equal scores by the LOWER index first (-0 and
    +0 are the same score);
  * keep the first min(k, nvis(t)); emit them in ascending index order and pad
    with -1 up to k.
"""
import numpy as np

from .indexer import nvis


def topk_row(scores_row, nv, k):
    """One row: scores_row [cap] (float), nv visible entries, k -> int32 [k]."""
    s = np.asarray(scores_row, dtype=np.float64)[:nv]
    e = np.arange(nv)
    # np.lexsort sorts by the last key first: primary -s (descending score),
    # secondary e (ascending index).  -0.0 and +0.0 compare equal.
    order = np.lexsort((e, -s))
    take = np.sort(order[: min(k, nv)])
    out = np.full(k, -1, dtype=np.int32)
    out[: take.size] = take
    return out


def topk(scores, q_pos0, m, k):
    """scores [B, T_q, cap] -> idx [B, T_q, k] int32."""
    scores = np.asarray(scores)
    B, T, cap = scores.shape
    out = np.empty((B, T, k), dtype=np.int32)
    for b in range(B):
        for i in range(T):
            nv = int(nvis(int(q_pos0[b]) + i, m))
            if nv > cap:
                raise ValueError("visible entries exceed the cache capacity")
            out[b, i] = topk_row(scores[b, i], nv, k)
    return out
