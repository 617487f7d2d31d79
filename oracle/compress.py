"""KV compression: one pooled entry per complete block of m tokens (test infrastructure).

Pages: CSA first compresses the KV cache so that every m tokens' key/value
pairs become one entry and the sequence shrinks to 1/m (blog.nickys.cn
DeepSeek-V4 post, 三大架构改动 §1 CSA; "DeepSeek-V4 技术分析报告" §3 架构层, CSA
bullet).  HCA does the same with a block m' far larger than m (blog.nickys.cn,
三大架构改动 §2 HCA).

Readings where the pages are silent:
  * The pooling rule is not given.  The project fixes it as a softmax-weighted
    pool with ONE scalar logit per token shared by K and V:
        a_j = exp(z_j - max z) / sum_i exp(z_i - max z),  Khat = sum_j a_j K_j,
        Vhat = sum_j a_j V_j.
    (parity unpinned by the pages: only the arithmetic below is pinned.)
  * Blocks are non-overlapping and aligned to position 0; a block exists only
    once complete, so L tokens give floor(L/m) entries.
  * Storage: bf16 or fp32 by round-to-nearest-even; or OCP E4M3FN with one
    fp32 scale per entry (separately for K and V): scale = fp32(amax / 448)
    (1 when amax == 0), code = RNE_e4m3(x / scale) saturated at +-448.
"""
import numpy as np

from .formats import bf16_encode, e4m3_encode, f32_round, E4M3_MAX


def pool_weights(z):
    """Softmax over the last axis in fp64, max-subtracted."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def compress_values(K, V, logits, m):
    """Exact-ish fp64 pooled entries before storage rounding.

    K, V: [B, L, d] float64; logits: [B, L] float64.  Returns (Khat, Vhat) of
    shape [B, floor(L/m), d] in float64.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    z = np.asarray(logits, dtype=np.float64)
    B, L, d = K.shape
    n = L // m
    Kb = K[:, : n * m].reshape(B, n, m, d)
    Vb = V[:, : n * m].reshape(B, n, m, d)
    a = pool_weights(z[:, : n * m].reshape(B, n, m))          # [B, n, m]
    Khat = np.einsum("bnm,bnmd->bnd", a, Kb)
    Vhat = np.einsum("bnm,bnmd->bnd", a, Vb)
    return Khat, Vhat


def fp8_quantize_entries(X):
    """Per-entry E4M3FN quantisation: returns (codes uint8 [.., d], scale fp32 [..])."""
    X = np.asarray(X, dtype=np.float64)
    amax = np.abs(X).max(axis=-1)
    scale = np.where(amax > 0, f32_round(amax / E4M3_MAX), 1.0)
    codes = e4m3_encode(X / scale[..., None])
    return codes, scale.astype(np.float32)


def store(X, out_dtype):
    """Round pooled fp64 values to the storage type.

    out_dtype: "bf16" -> uint16 bit patterns; "f32" -> float32;
    "fp8" -> (uint8 codes, float32 per-entry scale).
    """
    if out_dtype == "bf16":
        return bf16_encode(X)
    if out_dtype == "f32":
        return np.asarray(X, dtype=np.float64).astype(np.float32)
    if out_dtype == "fp8":
        return fp8_quantize_entries(X)
    raise ValueError(out_dtype)


def compress_kv(K, V, logits, m, out_dtype):
    """Full compression step: pooled entries stored in `out_dtype` (K then V)."""
    Khat, Vhat = compress_values(K, V, logits, m)
    return store(Khat, out_dtype), store(Vhat, out_dtype)
