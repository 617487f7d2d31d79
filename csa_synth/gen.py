"""Seeded input generators.

Every tensor comes from numpy PCG64 streams spawned from
SeedSequence([0xC5A, tag, seed]) in a fixed order, so any input can be
regenerated from (tag, seed) alone.  Distributions:
  * raw K / V / Q: N(0,1) drawn in fp32 and rounded to bf16 (fp32 variant:
    kept in fp32); optional outliers: each element independently with
    probability 0.01 is multiplied by 8;
  * pooling logits: fp32 N(0,1);
  * MXFP4 indexer operands: every E2M1 code (16 of them, -0 included) equally
    likely; block scales E8M0 uniform in {126, 127, 128} (2^-1, 2^0, 2^1);
  * indexer head weights w: uniform in {1/2, 1, 2};
  * pre-existing compressed caches (long prefixes) are drawn directly:
    bf16 / fp32 N(0,1) entries, or fp8 E4M3FN codes with one power-of-two fp32
    scale per entry chosen so the entry's largest magnitude fits in +-448.

With these, every indexer partial sum is an integer multiple of 2^-5 below
2^24 * 2^-5 in magnitude, so indexer scores are exact in fp32 in any
summation order (checked by the oracle tests).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_ROOT = 0xC5A
D = 128


def streams(tag, seed, n):
    ss = np.random.SeedSequence([SEED_ROOT, int(tag), int(seed)])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 bit patterns (nearest, ties to even; finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def normal_f32(rng, shape, outlier_rng=None, p=0.01, factor=8.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_rng is not None:
        x = np.where(outlier_rng.random(shape) < p, x * np.float32(factor), x)
    return x


def normal_kv(rng, shape, dtype, outlier_rng=None):
    """N(0,1) (+outliers) in the given storage dtype ('bf16' -> uint16 bits, 'f32')."""
    x = normal_f32(rng, shape, outlier_rng)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def fp8_entries(rng, shape, outlier_rng=None):
    """Directly drawn fp8 E4M3FN entries: (codes uint8 [..., d], scale float32 [...])."""
    import torch
    x = normal_f32(rng, shape, outlier_rng)
    amax = np.abs(x).max(axis=-1)
    scale = np.exp2(np.ceil(np.log2(np.maximum(amax, 1e-30) / 448.0))).astype(np.float32)
    y = torch.from_numpy(np.ascontiguousarray(x / scale[..., None]))
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def mxfp4_random(rng_codes, rng_exp, lead, d, codes=None, exps=(126, 127, 128)):
    """Random MXFP4 tensor: (packed uint8 [*lead, d/2], e8m0 uint8 [*lead, d/32]).

    codes: optional restricted set of 4-bit codes (default: all 16).
    """
    lead = tuple(lead)
    if codes is None:
        packed = rng_codes.integers(0, 256, lead + (d // 2,), dtype=np.uint8)
    else:
        nib = rng_codes.choice(np.asarray(codes, dtype=np.uint8), size=lead + (d,))
        packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    e8 = rng_exp.choice(np.asarray(exps, dtype=np.uint8), size=lead + (d // 32,))
    return packed, e8


def dyadic_w(rng, shape, values=(0.5, 1.0, 2.0)):
    return rng.choice(np.asarray(values, dtype=np.float32), size=shape)


# --------------------------------------------------------------------------
# Per-step input sets


def compress_inputs(B, L, in_dtype="bf16", seed=0, tag=1, outliers=False):
    rk, rv, rz, ro = streams(tag, seed, 4)
    orng = ro if outliers else None
    return dict(K=normal_kv(rk, (B, L, D), in_dtype, orng),
                V=normal_kv(rv, (B, L, D), in_dtype, orng),
                logits=rz.standard_normal((B, L), dtype=np.float32))


def indexer_inputs(B, T, cap, H_I, d_I, seed=0, tag=2, tie_heavy=False):
    """MXFP4 query / key operands and head weights.

    tie_heavy: codes restricted to {0, +1, -1}, all scales 2^0 and w = 1, so
    scores are small integers and the top-k boundary carries many ties.
    """
    rqc, rqe, rkc, rke, rw = streams(tag, seed, 5)
    if tie_heavy:
        codes, exps = (0, 2, 10), (127,)
    else:
        codes, exps = None, (126, 127, 128)
    qc, qe = mxfp4_random(rqc, rqe, (B, T, H_I), d_I, codes, exps)
    kc, ke = mxfp4_random(rkc, rke, (B, cap), d_I, codes, exps)
    w = (np.ones((B, T, H_I), np.float32) if tie_heavy else dyadic_w(rw, (B, T, H_I)))
    return dict(q_codes=qc, q_e8m0=qe, w=w, k_codes=kc, k_e8m0=ke)


def random_scores(B, T, cap, seed=0, tag=3, distinct=64):
    """fp32 score rows with many repeated values (drawn from `distinct` levels, +-0 mixed in)."""
    (r,) = streams(tag, seed, 1)
    levels = np.concatenate([[0.0, -0.0], r.standard_normal(distinct - 2)]).astype(np.float32)
    return levels[r.integers(0, distinct, (B, T, cap))]


def attn_inputs(B, T, H, cap, L_raw, io_dtype="bf16", ckv_dtype="bf16", seed=0, tag=4,
                outliers=False):
    """Query, compressed cache and raw window buffer for one attention call."""
    rq, rck, rcv, rkw, rvw, ro = streams(tag, seed, 6)
    orng = ro if outliers else None
    out = dict(q=normal_kv(rq, (B, T, H, D), io_dtype))
    if ckv_dtype == "fp8":
        out["cK"], out["cK_scale"] = fp8_entries(rck, (B, cap, D), orng)
        out["cV"], out["cV_scale"] = fp8_entries(rcv, (B, cap, D), orng)
    else:
        out["cK"] = normal_kv(rck, (B, cap, D), ckv_dtype, orng)
        out["cV"] = normal_kv(rcv, (B, cap, D), ckv_dtype, orng)
        out["cK_scale"] = out["cV_scale"] = None
    out["Kw"] = normal_kv(rkw, (B, L_raw, D), io_dtype, orng)
    out["Vw"] = normal_kv(rvw, (B, L_raw, D), io_dtype, orng)
    return out


def random_topk_idx(nv, k, cap, seed=0, tag=5):
    """idx [B, T, k]: per row, min(k, nv) distinct indices < nv ascending, then -1.

    nv: int array [B, T] of visible-entry counts (passed in by the caller).
    """
    (r,) = streams(tag, seed, 1)
    nv = np.asarray(nv)
    B, T = nv.shape
    out = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for i in range(T):
            n = int(min(nv[b, i], cap))
            c = min(k, n)
            if c:
                out[b, i, :c] = np.sort(r.choice(n, size=c, replace=False))
    return out


# --------------------------------------------------------------------------
# Workloads (shapes of the pages' 4K - 1M contexts)


@dataclass
class Workload:
    name: str
    B: int
    T_q: int
    H: int
    m: int                  # CSA block (or HCA block for kind == "hca")
    W: int
    kind: str               # "csa" or "hca"
    ckv: str                # compressed-cache storage: bf16 | f32 | fp8
    q_pos0: list            # absolute position of query 0, per sequence
    cap: int                # compressed entries per sequence in the cache
    L_raw: int              # rows of the raw window buffer
    raw_pos0: list          # absolute position of raw row 0, per sequence
    k: int = 0
    H_I: int = 0
    d_I: int = 0
    outliers: bool = False
    tag: int = 0
    extra: dict = field(default_factory=dict)


def decode_workload(name, B, n, H, m, W, kind, ckv, k=0, H_I=0, d_I=0, outliers=False, tag=0):
    """B sequences with context n each (the query is the n-th token, at position n-1)."""
    L_raw = W
    return Workload(name, B, 1, H, m, W, kind, ckv, [n - 1] * B, n // m, L_raw,
                    [n - L_raw] * B, k, H_I, d_I, outliers, tag)


def prefill_workload(name, P, C, H, m, W, kind, ckv, k=0, H_I=0, d_I=0, outliers=False, tag=0):
    """One sequence: C new queries at positions P .. P+C-1 (their K/V already in the cache)."""
    L_raw = C + W
    return Workload(name, 1, C, H, m, W, kind, ckv, [P], (P + C) // m, L_raw, [P + C - L_raw],
                    k, H_I, d_I, outliers, tag)


def workloads():
    """The five workload shapes (tiny decode, 128K CSA decode, 1M HCA decode, CSA prefill
    chunk at 256K, and the 1M layer pair split into its four calls)."""
    return {
        "tiny_csa_decode_4k": decode_workload("tiny_csa_decode_4k", 1, 4096, 16, 4, 128, "csa",
                                              "bf16", k=64, H_I=4, d_I=64, tag=11),
        "csa_decode_128k": decode_workload("csa_decode_128k", 16, 131072, 64, 4, 128, "csa",
                                           "bf16", k=1024, H_I=8, d_I=128, tag=12),
        "hca_decode_1m": decode_workload("hca_decode_1m", 4, 1048576, 64, 128, 128, "hca", "fp8",
                                         tag=13),
        "csa_prefill_256k": prefill_workload("csa_prefill_256k", 262144, 4096, 64, 4, 128, "csa",
                                             "bf16", k=2048, H_I=8, d_I=128, tag=14),
        "pair_csa_decode_1m": decode_workload("pair_csa_decode_1m", 4, 1048576, 64, 4, 128, "csa",
                                              "fp8", k=1024, H_I=8, d_I=128, outliers=True,
                                              tag=15),
        "pair_csa_chunk_1m": prefill_workload("pair_csa_chunk_1m", 1048576, 2048, 64, 4, 128,
                                              "csa", "fp8", k=1024, H_I=8, d_I=128,
                                              outliers=True, tag=16),
        "pair_hca_decode_1m": decode_workload("pair_hca_decode_1m", 4, 1048576, 64, 128, 128,
                                              "hca", "fp8", outliers=True, tag=17),
        "pair_hca_chunk_1m": prefill_workload("pair_hca_chunk_1m", 1048576, 2048, 64, 128, 128,
                                              "hca", "fp8", outliers=True, tag=18),
    }
