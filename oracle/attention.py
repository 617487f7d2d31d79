"""CSA sparse attention and HCA dense attention, each with the window branch.

Test infrastructure.  Pages:
  * CSA attends only over the k selected compressed entries and additionally
    keeps a few uncompressed sliding-window entries so short-range dependencies
    are not lost (blog.nickys.cn DeepSeek-V4 post, 三大架构改动 §1 CSA;
    "DeepSeek-V4 技术分析报告" §3 架构层, 滑动窗口分支 bullet).
  * HCA does no sparse selection and attends densely over ALL compressed
    entries (blog.nickys.cn, 三大架构改动 §2 HCA).
  * Both kinds add the window branch so every token fully sees its nearest
    neighbours (sz-guanghua.com.cn ifanr repost, 百萬長上下文 section).

Readings where the pages are silent:
  * window(t) = positions [max(0, t - W + 1), t], the token itself included;
  * the selected (or all visible) compressed entries and the window keys form
    ONE key set under one softmax, concatenated with no de-duplication (the
    window is an additional branch);
  * logit = sm * (q_h . key) with sm = 1/sqrt(d) unless given; no sink, no
    bias; inputs are taken as already position-encoded;
  * an empty key set gives O = 0 and lse = -inf;
  * all query heads share the one KV head (the compressed entry / raw token).
"""
import math

import numpy as np

from .formats import bf16_decode, e4m3_decode
from .indexer import nvis


def decode_kv(arr, dtype, scale=None):
    """Stored KV -> float64.  dtype: 'bf16' (uint16 bits), 'f32', or 'fp8' (codes, per-entry scale)."""
    if dtype == "bf16":
        return bf16_decode(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_decode(arr) * np.asarray(scale, dtype=np.float64)[..., None]
    raise ValueError(dtype)


def softmax_attend(qh, keys, vals, sm):
    """One query, all heads: qh [H, d], keys/vals [n, d] -> (O [H, d], lse [H])."""
    H, d = qh.shape
    if keys.shape[0] == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    logit = sm * (qh @ keys.T)                     # [H, n]
    mx = logit.max(axis=1, keepdims=True)
    p = np.exp(logit - mx)
    s = p.sum(axis=1, keepdims=True)
    P = p / s
    return P @ vals, (mx + np.log(s))[:, 0]


def window_rows(t, W, raw_pos0, L_raw):
    """Raw-buffer rows of window(t).  The buffer must cover the whole window."""
    lo = max(0, t - W + 1)
    pos = np.arange(lo, t + 1)
    rows = pos - raw_pos0
    if rows.size and (rows[0] < 0 or rows[-1] >= L_raw):
        raise ValueError("raw window buffer does not cover the window")
    return rows


def sparse_attn(q, cK, cV, idx, Kw, Vw, raw_pos0, q_pos0, W, sm=None):
    """CSA attention.

    q [B,T,H,d]; cK, cV [B,cap,d]; idx [B,T,k] (-1 = empty slot);
    Kw, Vw [B,L_raw,d] raw window buffer whose row r is position raw_pos0[b]+r.
    All float arrays are float64 values.  Returns (O [B,T,H,d], lse [B,T,H]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, H, d = q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else sm
    O = np.zeros((B, T, H, d))
    lse = np.zeros((B, T, H))
    L_raw = Kw.shape[1]
    for b in range(B):
        for i in range(T):
            t = int(q_pos0[b]) + i
            sel = [int(e) for e in idx[b, i] if e >= 0]
            rows = window_rows(t, W, int(raw_pos0[b]), L_raw)
            keys = np.concatenate([cK[b, sel], Kw[b, rows]], axis=0)
            vals = np.concatenate([cV[b, sel], Vw[b, rows]], axis=0)
            O[b, i], lse[b, i] = softmax_attend(q[b, i], keys, vals, sm)
    return O, lse


def dense_attn(q, cK, cV, m_prime, Kw, Vw, raw_pos0, q_pos0, W, sm=None):
    """HCA attention: every visible compressed entry e < floor((t+1)/m') plus window(t)."""
    q = np.asarray(q, dtype=np.float64)
    B, T, H, d = q.shape
    sm = 1.0 / math.sqrt(d) if sm is None else sm
    O = np.zeros((B, T, H, d))
    lse = np.zeros((B, T, H))
    cap = cK.shape[1]
    L_raw = Kw.shape[1]
    for b in range(B):
        for i in range(T):
            t = int(q_pos0[b]) + i
            nv = int(nvis(t, m_prime))
            if nv > cap:
                raise ValueError("visible entries exceed the cache capacity")
            rows = window_rows(t, W, int(raw_pos0[b]), L_raw)
            keys = np.concatenate([cK[b, :nv], Kw[b, rows]], axis=0)
            vals = np.concatenate([cV[b, :nv], Vw[b, rows]], axis=0)
            O[b, i], lse[b, i] = softmax_attend(q[b, i], keys, vals, sm)
    return O, lse


def layer_pair(csa_inputs, hca_inputs):
    """An interleaved CSA layer followed by an HCA layer.

    Different layers use different attention kinds and the two kinds are
    interleaved ("DeepSeek-V4 技术分析报告" §3 架构层; blog.nickys.cn
    三大架构改动 §2 HCA).  Projections between layers are outside the path, so
    the two calls share no data: each gets its own inputs (dicts of the
    keyword arguments of sparse_attn / dense_attn).
    """
    return sparse_attn(**csa_inputs), dense_attn(**hca_inputs)
