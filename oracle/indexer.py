"""Lightning-indexer scores on MXFP4 operands (test infrastructure).

Pages: a lightweight "Lightning Indexer" picks, for the current query, the k
compressed KV entries most relevant to it (blog.nickys.cn DeepSeek-V4 post,
三大架构改动 §1 CSA); it uses FP4 to score every query token against every
compressed block (sz-guanghua.com.cn ifanr repost, 百萬長上下文 section); the FP4
format on the indexer's query-key path is MXFP4 ("DeepSeek V4技术揭秘", §一).

Reading fixed by the project (parity unpinned by the pages): the score of
entry e for the query at absolute position t is
    s(t, e) = sum_h w[t, h] * max(0, q[t, h] . k[e])
with one MXFP4 key vector per entry shared by all indexer heads (supplied by
the caller) and a per-query, per-head weight w.  Causality: entry e covers
positions [e*m, (e+1)*m) and is visible at t iff the whole block is <= t,
i.e. e < nvis(t) = floor((t + 1) / m); other entries score -inf.
"""
import numpy as np

from .formats import mxfp4_decode


def nvis(t, m):
    """Number of compressed entries whose whole block lies at or before t."""
    return (np.asarray(t, dtype=np.int64) + 1) // m


def indexer_scores(q_codes, q_e8m0, w, k_codes, k_e8m0, q_pos0, m, check_exact=True):
    """Scores [B, T_q, cap] as float64 (-inf where not visible).

    q_codes [B,T,H,d/2] u8, q_e8m0 [B,T,H,d/32] u8, w [B,T,H] (float),
    k_codes [B,cap,d/2] u8, k_e8m0 [B,cap,d/32] u8, q_pos0 [B] int.
    With check_exact the function asserts that every visible score is exactly
    representable in fp32 (which the input generator is built to guarantee),
    so the fp32 cast of the result is the exact score.
    """
    Q = mxfp4_decode(q_codes, q_e8m0)                # [B, T, H, dI]
    Kx = mxfp4_decode(k_codes, k_e8m0)               # [B, cap, dI]
    w = np.asarray(w, dtype=np.float64)
    B, T, H, dI = Q.shape
    cap = Kx.shape[1]
    out = np.full((B, T, cap), -np.inf)
    for b in range(B):
        dots = np.einsum("thi,ei->the", Q[b], Kx[b])  # [T, H, cap]
        s = np.einsum("th,the->te", w[b], np.maximum(dots, 0.0))
        t = int(q_pos0[b]) + np.arange(T)
        nv = nvis(t, m)
        if np.any(nv > cap):
            raise ValueError("visible entries exceed the cache capacity")
        vis = np.arange(cap)[None, :] < nv[:, None]
        out[b][vis] = s[vis]
    if check_exact:
        fin = np.isfinite(out)
        if not np.array_equal(out[fin].astype(np.float32).astype(np.float64), out[fin]):
            raise AssertionError("indexer score not exactly representable in fp32")
    return out
