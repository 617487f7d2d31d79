"""Benchmark of the CSA / HCA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input.  The
default run (--workload all) measures four full-size workloads, one after the
other, and prints them in ONE JSON line:
  * headline (value, steps, ms_per_step, roofline, cpu_baseline): the 1M-context
    CSA + HCA layer pair -- a CSA layer (4 decode rows at 1M with 262144 fp8
    entries, then a 2048-token chunk over 262656) followed by an HCA layer
    (8192 / 8208 fp8 entries), 2052 query tokens per step;
  * under "workloads": CSA decoding at 128K (16 sequences: pool the block the
    query completes, MXFP4 indexer over 32768 entries, top-1024, 64-head
    attention over them plus the 128-token window), HCA decoding at 1M (4
    sequences, 8192 fp8 entries + window) and CSA prefill of a 4096-token chunk
    at 256K (66560 entries, top-2048).
--workload picks one of them (or the quantiser / cache-append workloads) alone.

Inputs are resident in HBM before timing.  Each input copy's step is captured
into a HIP graph; copies rotate so that one rotation touches well over twice
the 256 MB Infinity Cache and reads are served by HBM.  Exactly --steps steps
are timed between two HIP events (after --warmup untimed ones); the median /
p10 / p90 of the step time come from --dist-steps replays of the all-copies
step graph, timed one by one.  Per-call
durations come from HIP events around graph replays of each call alone on the
stream it runs on.  The CPU oracle is timed on a bounded sample of the headline
workload on the host's cores.

Prints ONE JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA attention query-tokens/sec at 128K-1M ctx; % HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0
MXFP4_PEAK_TFLOPS = 10100.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="all",
                   choices=["all", "csa_decode_128k", "hca_decode_1m", "csa_prefill_256k", "pair_1m", "pair_1m_split",
                            "mxfp4_quantize_keys_128k", "kv_append_decode_128k"],
                   help="all (default): the 1M layer pair's mixed step (packed varlen calls) as the "
                        "headline line, with the 128K CSA decode, 1M HCA decode, 256K CSA prefill and "
                        "the pair's split-call step carried in it")
    p.add_argument("--dist-steps", type=int, default=100,
                   help="replays of the all-copies step graph, each timed alone, for the median / p10 / p90")
    p.add_argument("--rotate", type=int, default=0, help="input copies (0 = auto)")
    p.add_argument("--indexer", default="auto", choices=["auto", "combined", "fused", "unfused"],
                   help="CSA scoring + selection as one fused call or as csa_indexer_scores then "
                        "csa_topk (auto: fused for prefill chunks, unfused for decode)")
    p.add_argument("--batch-invariant", action="store_true",
                   help="attention through the batch-invariant calls (row bits independent of the batch)")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run 10 plain device copies of 256 MiB (reference for HBM byte counters)")
    return p.parse_args()


# --------------------------------------------------------------------------
# Workload construction (device tensors)

class Kernel:
    """One ABI call of a step: fn(copy), its algorithmic bytes and flops, and the peak
    of the unit its flops run on (MXFP4 or bf16 matrix cores)."""

    def __init__(self, name, fn, nbytes, flops, mfma_peak, src, hip=""):
        self.name, self.fn, self.nbytes, self.flops = name, fn, int(nbytes), int(flops)
        self.mfma_peak, self.src, self.hip = mfma_peak, src, hip

    @property
    def bound(self):
        """The roofline that bounds the call: the larger of bytes/HBM peak and flops/MFMA peak."""
        t_mem = self.nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = self.flops / (self.mfma_peak * 1e12) if self.flops else 0.0
        return "mfma" if t_mfma > t_mem else "hbm"


class Step:
    """One workload: device inputs (R rotating copies) and the launches of one step."""

    def __init__(self, name, q_tokens):
        self.name = name
        self.q_tokens = q_tokens
        self.copies = []
        self.kernels = {}
        self.order = []
        self.config = {}
        self.layers = []      # host inputs per layer, for the CPU baseline

    def add(self, k):
        self.kernels[k.name] = k
        self.order.append(k.name)

    def run(self, c):
        for n in self.order:
            self.kernels[n].fn(c)


def _t(x, kind):
    import torch
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    if kind == "u8":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8))
    if kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if kind == "i32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32))
    raise ValueError(kind)


def host_layer(wl, seed=0):
    """Host inputs of one layer's calls for workload wl (a csa_synth Workload)."""
    from csa_synth import attn_inputs, compress_inputs, indexer_inputs
    h = {"wl": wl}
    h["kv"] = compress_inputs(wl.B, wl.L_raw, "bf16", seed=seed, tag=wl.tag * 10 + 1,
                              outliers=wl.outliers)
    h["at"] = attn_inputs(wl.B, wl.T_q, wl.H, wl.cap, 1, "bf16", wl.ckv, seed=seed,
                          tag=wl.tag * 10 + 3, outliers=wl.outliers)
    if wl.kind == "csa":
        h["ix"] = indexer_inputs(wl.B, wl.T_q, wl.cap, wl.H_I, wl.d_I, seed=seed,
                                 tag=wl.tag * 10 + 2)
    return h


def pool_range(wl):
    """(rows pooled, first raw row, first entry written) of the step's compression: the block
    a decode query completes, or every block of a prefill chunk."""
    L = wl.T_q if wl.T_q > 1 else wl.m
    entry0 = (wl.q_pos0[0] + wl.T_q) // wl.m - L // wl.m
    return L, wl.L_raw - L, entry0


def device_layer(h, prefix):
    """Host arrays of one layer -> dict of CPU tensors keyed prefix+name."""
    import torch
    wl, kv, at = h["wl"], h["kv"], h["at"]
    T = dict(kw=_t(kv["K"], "bf16"), vw=_t(kv["V"], "bf16"), logits=_t(kv["logits"], "f32"),
             q=_t(at["q"], "bf16"), pos=_t(np.array(wl.q_pos0), "i32"),
             raw0=_t(np.array(wl.raw_pos0), "i32"),
             out=torch.empty((wl.B, wl.T_q, wl.H, 128), dtype=torch.bfloat16))
    if wl.ckv == "fp8":
        T.update(ck=_t(at["cK"], "u8"), cv=_t(at["cV"], "u8"), cks=_t(at["cK_scale"], "f32"),
                 cvs=_t(at["cV_scale"], "f32"))
    else:
        T.update(ck=_t(at["cK"], "bf16"), cv=_t(at["cV"], "bf16"), cks=None, cvs=None)
    if wl.kind == "csa":
        ix = h["ix"]
        T.update(qc=_t(ix["q_codes"], "u8"), qe=_t(ix["q_e8m0"], "u8"), w=_t(ix["w"], "f32"),
                 kc=_t(ix["k_codes"], "u8"), ke=_t(ix["k_e8m0"], "u8"),
                 scores=torch.empty((wl.B, wl.T_q, wl.cap), dtype=torch.float32),
                 idx=torch.empty((wl.B, wl.T_q, wl.k), dtype=torch.int32))
    return {prefix + n: v for n, v in T.items()}


def visible(wl):
    """Visible compressed entries summed over the step's query rows."""
    t = np.asarray(wl.q_pos0)[:, None] + np.arange(wl.T_q)[None, :]
    return int(np.minimum((t + 1) // wl.m, wl.cap).sum())


def add_layer(st, h, prefix, indexer="auto", batch_invariant=False):
    """The calls of one CSA or HCA layer: compress, (indexer, top-k,) attention."""
    import long_context_compressed_03_amd as csa
    wl = h["wl"]
    p = prefix
    B, m, W, H, rows = wl.B, wl.m, wl.W, wl.H, wl.B * wl.T_q
    L, row0, entry0 = pool_range(wl)
    ent = 264 if wl.ckv == "fp8" else 512
    nvis_sum = visible(wl)
    name = (lambda n: f"{prefix}{n}") if prefix else (lambda n: n)

    def f_compress(c):
        csa.csa_compress_kv(c[p + "kw"], c[p + "vw"], c[p + "logits"], m, c[p + "ck"], c[p + "cv"],
                            c[p + "cks"], c[p + "cvs"], L=L, row0=row0, entry0=entry0)
    compress_bytes = B * (L * 516 + (L // m) * ent)
    decode_split = wl.kind == "csa" and wl.T_q == 1 and rows <= 128 and wl.cap >= 8192 and wl.d_I <= 256
    # decoding: the compression rides in the indexer top-k call (one launch fewer)
    combined = decode_split and m < 32 and indexer in ("auto", "combined")
    if not combined:
        st.add(Kernel(name("compress_kv"), f_compress, compress_bytes, 0, BF16_PEAK_TFLOPS, "compress_kv",
                      "compress_long_kernel" if m >= 32 else "compress_kernel"))
    q_bytes = rows * H * 128 * 4          # bf16 query in + bf16 output
    if wl.kind == "csa":
        k = wl.k
        idx_bytes = wl.d_I // 2 + wl.d_I // 32

        def f_indexer(c):
            csa.csa_indexer_scores(c[p + "qc"], c[p + "qe"], c[p + "w"], c[p + "kc"], c[p + "ke"],
                                   c[p + "pos"], m, c[p + "scores"])

        def f_topk(c):
            csa.csa_topk(c[p + "scores"], c[p + "pos"], m, k, c[p + "idx"])

        def f_attn(c):
            csa.csa_sparse_attn(c[p + "q"], c[p + "ck"], c[p + "cv"], c[p + "idx"], c[p + "kw"],
                                c[p + "vw"], c[p + "raw0"], c[p + "pos"], W, ck_scale=c[p + "cks"],
                                cv_scale=c[p + "cvs"], out=c[p + "out"], batch_invariant=batch_invariant)
        fused = indexer in ("fused", "auto", "combined")
        if combined:
            def f_combined(c):
                csa.csa_compress_indexer_topk(c[p + "kw"], c[p + "vw"], c[p + "logits"], c[p + "ck"],
                                              c[p + "cv"], c[p + "cks"], c[p + "cvs"], c[p + "qc"],
                                              c[p + "qe"], c[p + "w"], c[p + "kc"], c[p + "ke"],
                                              c[p + "pos"], m, k, idx=c[p + "idx"], L=L, row0=row0,
                                              entry0=entry0)
            # keys once, the fp32 scores written, the indices; plus the compression's rows and entries
            st.add(Kernel(name("compress_indexer_topk"), f_combined,
                          compress_bytes + B * wl.cap * idx_bytes + nvis_sum * 4 + rows * k * 4
                          + rows * wl.H_I * (idx_bytes + 4),
                          2 * wl.H_I * wl.d_I * nvis_sum, MXFP4_PEAK_TFLOPS, "compress_indexer_topk",
                          "indexer_slice_kernel, topk_kernel<true> (with the compression blocks)"))
        elif fused:
            def f_fused(c):
                csa.csa_indexer_topk(c[p + "qc"], c[p + "qe"], c[p + "w"], c[p + "kc"], c[p + "ke"],
                                     c[p + "pos"], m, k, c[p + "idx"])
            if decode_split:
                # decoding: keys once, the fp32 scores written (read back only by the
                # exact fallback), the indices
                inter = nvis_sum * 4
            else:
                # keys once; the sampled 16-bit keys written and read back; the
                # candidate (key, entry) pairs, about 2k per row, written and read back
                inter = tile_inter_bytes(rows, wl.cap, k)
            st.add(Kernel(name("indexer_topk"), f_fused,
                          B * wl.cap * idx_bytes + inter + rows * k * 4 + rows * wl.H_I * (idx_bytes + 4),
                          2 * wl.H_I * wl.d_I * nvis_sum, MXFP4_PEAK_TFLOPS, "indexer_topk",
                          "indexer_slice_kernel, topk_kernel<true>" if decode_split else TILE_TOPK_HIP))
        else:
            st.add(Kernel(name("indexer_scores"), f_indexer,
                          B * wl.cap * idx_bytes + rows * wl.cap * 4 + rows * wl.H_I * (idx_bytes + 4),
                          2 * wl.H_I * wl.d_I * nvis_sum, MXFP4_PEAK_TFLOPS, "indexer_scores", "indexer_kernel"))
            st.add(Kernel(name("topk"), f_topk, nvis_sum * 4 + rows * k * 4, 0, BF16_PEAK_TFLOPS,
                          "topk", "slice_select_kernel, topk_kernel<true>" if decode_split else "topk_kernel"))
        # distinct bytes: every selected entry at most once per sequence, the window rows once
        sel = min(B * wl.cap, rows * k)
        st.add(Kernel(name("sparse_attn"), f_attn,
                      sel * ent + B * wl.L_raw * 512 + q_bytes + rows * k * 4,
                      4 * H * 128 * rows * (k + W), BF16_PEAK_TFLOPS, "sparse_attn", attn_hip(rows, False, wl.T_q)))
    else:
        def f_attn(c):
            csa.hca_dense_attn(c[p + "q"], c[p + "ck"], c[p + "cv"], m, c[p + "kw"], c[p + "vw"],
                               c[p + "raw0"], c[p + "pos"], W, ck_scale=c[p + "cks"],
                               cv_scale=c[p + "cvs"], out=c[p + "out"], batch_invariant=batch_invariant)
        nv_max = min((wl.q_pos0[0] + wl.T_q) // m, wl.cap)
        st.add(Kernel(name("dense_attn"), f_attn, B * nv_max * ent + B * wl.L_raw * 512 + q_bytes,
                      4 * H * 128 * (nvis_sum + rows * W), BF16_PEAK_TFLOPS, "dense_attn", attn_hip(rows, True, wl.T_q)))


# Kernels of the row-tile indexer top-k (threshold path; the 16-bit-key pass and
# select_kernel sit behind the miss gate and return at once unless a row missed)
TILE_TOPK_HIP = ("indexer_kernel (sample, candidates), cand_threshold_kernel, cand_select_kernel; "
                 "indexer_kernel (16-bit keys), select_kernel behind the miss gate")


def tile_inter_bytes(rows, cap, k):
    """Bytes the threshold path moves besides the keys and indices: every row's sampled
    16-bit keys (16 of every 1024 entries) written and read back, and its candidate
    (key, entry) pairs, about 2k per row, written and read back."""
    if not (k <= 3276 and 32768 < cap <= (1 << 19)):
        # outside the threshold path's range: 16-bit keys of every entry written and read
        return rows * cap * 2 * 2
    sampled = (cap // 1024) * 16 + min(cap % 1024, 16)
    return rows * sampled * 2 * 2 + rows * 2 * k * 8 * 2


def attn_hip(rows, dense, T_q):
    """HIP kernels of an attention call: key lists are split over blocks (and merged by a
    second kernel) when the rows alone do not fill the chip; dense chunks of 64 queries or
    more take the many-query kernel."""
    if rows < 256:
        return "attn_kernel, attn_merge_kernel"
    return "attn_mq_kernel" if dense and T_q >= 64 else "attn_kernel"


def layer_config(wl):
    c = {"batch": wl.B, "query_tokens_per_seq": wl.T_q, "context": wl.q_pos0[0] + wl.T_q,
         "query_heads": wl.H, "kv_heads": 1, "head_dim": 128, "compressed_entries": wl.cap,
         "window": wl.W, "window_kv": "bf16",
         "compressed_kv": "fp8_e4m3+fp32 scale" if wl.ckv == "fp8" else wl.ckv}
    if wl.kind == "csa":
        c.update(m=wl.m, indexer=f"{wl.H_I}x{wl.d_I} MXFP4", top_k=wl.k)
    else:
        c.update(m_prime=wl.m)
    if wl.outliers:
        c["outliers"] = "1% x8"
    return c


LAYERS = {
    "csa_decode_128k": [("", "csa_decode_128k")],
    "hca_decode_1m": [("", "hca_decode_1m")],
    "csa_prefill_256k": [("", "csa_prefill_256k")],
    "pair_1m_split": [("csa_decode.", "pair_csa_decode_1m"), ("csa_chunk.", "pair_csa_chunk_1m"),
                      ("hca_decode.", "pair_hca_decode_1m"), ("hca_chunk.", "pair_hca_chunk_1m")],
}


def pack_layer(dec, ch):
    """One layer of the mixed step: the decode sequences' and the chunk's host inputs packed
    into one batch of B_dec + 1 sequences (caches padded to the larger capacity, raw windows
    to the chunk's length with every sequence's newest token in the last row) and query rows
    packed decode rows first."""
    wd, wc = dec["wl"], ch["wl"]
    nd, B = wd.B, wd.B + 1
    L_raw, cap = max(wd.L_raw, wc.L_raw), max(wd.cap, wc.cap)
    off = L_raw - wd.L_raw

    def raw(key, dt, extra=()):
        a = np.zeros((B, L_raw) + extra, dt)
        a[:nd, off:] = dec["kv"][key]
        a[nd, L_raw - wc.L_raw:] = ch["kv"][key][0]
        return a

    def cache(src, key, dt, extra):
        a = np.zeros((B, cap) + extra, dt)
        a[:nd, :wd.cap] = dec[src][key]
        a[nd, :wc.cap] = ch[src][key][0]
        return a
    p = {"K": raw("K", np.uint16, (128,)), "V": raw("V", np.uint16, (128,)), "logits": raw("logits", np.float32),
         "raw0": np.array([r - off for r in wd.raw_pos0] + [wc.raw_pos0[0] - (L_raw - wc.L_raw)], np.int32),
         "q": np.concatenate([dec["at"]["q"][:, 0], ch["at"]["q"][0]]), "L_raw": L_raw, "cap": cap}
    ckv = wd.ckv
    ext = (128,)
    p["cK"] = cache("at", "cK", np.uint8 if ckv == "fp8" else np.uint16, ext)
    p["cV"] = cache("at", "cV", np.uint8 if ckv == "fp8" else np.uint16, ext)
    if ckv == "fp8":
        p["cK_scale"] = cache("at", "cK_scale", np.float32, ())
        p["cV_scale"] = cache("at", "cV_scale", np.float32, ())
    n_rows = nd + wc.T_q
    p["pos0"] = np.array(list(wd.q_pos0) + [wc.q_pos0[0]], np.int32)
    p["cu_rows"] = np.array(list(range(nd + 1)) + [n_rows], np.int32)
    # the blocks the step completes: the decode tokens' (pool_range) and the chunk's
    Ld, r0d, e0d = pool_range(wd)
    Lc, r0c, e0c = pool_range(wc)
    n_d, n_c = Ld // wd.m, Lc // wc.m
    p["cu_entries"] = np.array([i * n_d for i in range(nd + 1)] + [nd * n_d + n_c], np.int32)
    p["row0"] = np.array([r0d + off] * nd + [r0c + (L_raw - wc.L_raw)], np.int32)
    p["entry0"] = np.array([e0d] * nd + [e0c], np.int32)
    p["n_entries"] = nd * n_d + n_c
    if wd.kind == "csa":
        for key in ("q_codes", "q_e8m0", "w"):
            p[key] = np.concatenate([dec["ix"][key][:, 0], ch["ix"][key][0]])
        p["k_codes"] = cache("ix", "k_codes", np.uint8, (wd.d_I // 2,))
        p["k_e8m0"] = cache("ix", "k_e8m0", np.uint8, (wd.d_I // 32,))
    return p


def add_varlen_layer(st, dec, ch, prefix):
    """The mixed step's calls of one layer: compression, (indexer top-k,) attention, each one
    launch over all the step's sequences."""
    import long_context_compressed_03_amd as csa
    wd, wc = dec["wl"], ch["wl"]
    p, m, W, H = prefix, wd.m, wd.W, wd.H
    nd = wd.B
    rows = nd + wc.T_q
    ent = 264 if wd.ckv == "fp8" else 512
    Ld, Lc = pool_range(wd)[0], pool_range(wc)[0]
    nvis_d, nvis_c = visible(wd), visible(wc)

    def f_compress(c):
        csa.csa_compress_kv_varlen(c[p + "kw"], c[p + "vw"], c[p + "logits"], m, c[p + "ck"], c[p + "cv"],
                                   c[p + "cu_entries"], c[p + "row0"], c[p + "entry0"], c[p + "n_entries"],
                                   k_scale_out=c[p + "cks"], v_scale_out=c[p + "cvs"])
    st.add(Kernel(p + "compress_kv", f_compress, nd * (Ld * 516 + (Ld // m) * ent) + Lc * 516 + (Lc // m) * ent, 0,
                  BF16_PEAK_TFLOPS, "compress_kv", "compress_long_kernel" if m >= 32 else "compress_kernel"))
    q_bytes = rows * H * 128 * 4
    if wd.kind == "csa":
        k = wd.k
        idx_bytes = wd.d_I // 2 + wd.d_I // 32
        cap = max(wd.cap, wc.cap)

        def f_sel(c):
            csa.csa_indexer_topk_varlen(c[p + "qc"], c[p + "qe"], c[p + "w"], c[p + "kc"], c[p + "ke"],
                                        c[p + "cu_rows"], c[p + "pos"], m, k, c[p + "idx"])
        # each sequence's keys once, the sample and candidate traffic of the threshold
        # path, the indices, the queries and weights
        st.add(Kernel(p + "indexer_topk", f_sel,
                      (nd * wd.cap + wc.cap) * idx_bytes + tile_inter_bytes(rows, cap, k) + rows * k * 4
                      + rows * wd.H_I * (idx_bytes + 4),
                      2 * wd.H_I * wd.d_I * (nvis_d + nvis_c), MXFP4_PEAK_TFLOPS, "indexer_topk",
                      TILE_TOPK_HIP))

        def f_attn(c):
            csa.csa_sparse_attn_varlen(c[p + "q"], c[p + "ck"], c[p + "cv"], c[p + "idx"], c[p + "kw"], c[p + "vw"],
                                       c[p + "raw0"], c[p + "cu_rows"], c[p + "pos"], W, ck_scale=c[p + "cks"],
                                       cv_scale=c[p + "cvs"], invariant=False, out=c[p + "out"])
        sel = min(nd * wd.cap, nd * k) + min(wc.cap, wc.T_q * k)
        st.add(Kernel(p + "sparse_attn", f_attn,
                      sel * ent + (nd * wd.L_raw + wc.L_raw) * 512 + q_bytes + rows * k * 4,
                      4 * H * 128 * rows * (k + W), BF16_PEAK_TFLOPS, "sparse_attn", "attn_kernel"))
    else:
        def f_attn(c):
            csa.hca_dense_attn_varlen(c[p + "q"], c[p + "ck"], c[p + "cv"], m, c[p + "kw"], c[p + "vw"], c[p + "raw0"],
                                      c[p + "cu_rows"], c[p + "pos"], W, ck_scale=c[p + "cks"],
                                      cv_scale=c[p + "cvs"], invariant=False, out=c[p + "out"])
        nv_d = min((wd.q_pos0[0] + 1) // m, wd.cap)
        nv_c = min((wc.q_pos0[0] + wc.T_q) // m, wc.cap)
        st.add(Kernel(p + "dense_attn", f_attn,
                      (nd * nv_d + nv_c) * ent + (nd * wd.L_raw + wc.L_raw) * 512 + q_bytes,
                      4 * H * 128 * (nvis_d + nvis_c + rows * W), BF16_PEAK_TFLOPS, "dense_attn",
                      "attn_mq_kernel, attn_merge_kernel"))


def device_packed(pk, prefix, kind, k=0):
    """Packed host arrays of one layer -> dict of CPU tensors keyed prefix+name."""
    import torch
    T = dict(kw=_t(pk["K"], "bf16"), vw=_t(pk["V"], "bf16"), logits=_t(pk["logits"], "f32"),
             q=_t(pk["q"], "bf16"), pos=_t(pk["pos0"], "i32"), raw0=_t(pk["raw0"], "i32"),
             cu_rows=_t(pk["cu_rows"], "i32"),
             cu_entries=_t(pk["cu_entries"], "i32"), row0=_t(pk["row0"], "i32"), entry0=_t(pk["entry0"], "i32"),
             n_entries=int(pk["n_entries"]),
             out=torch.empty(pk["q"].shape, dtype=torch.bfloat16))
    if "cK_scale" in pk:
        T.update(ck=_t(pk["cK"], "u8"), cv=_t(pk["cV"], "u8"), cks=_t(pk["cK_scale"], "f32"),
                 cvs=_t(pk["cV_scale"], "f32"))
    else:
        T.update(ck=_t(pk["cK"], "bf16"), cv=_t(pk["cV"], "bf16"), cks=None, cvs=None)
    if kind == "csa":
        T.update(qc=_t(pk["q_codes"], "u8"), qe=_t(pk["q_e8m0"], "u8"), w=_t(pk["w"], "f32"),
                 kc=_t(pk["k_codes"], "u8"), ke=_t(pk["k_e8m0"], "u8"),
                 idx=torch.empty((pk["q"].shape[0], k), dtype=torch.int32))
    return {prefix + n: v for n, v in T.items()}


QUANT_WORKLOAD = "mxfp4_quantize_keys_128k"
QUANT_SHAPE = (16 * 32768, 128)     # the 128K decode shape's indexer keys


def build_quant(args):
    """The MXFP4 quantisation of the indexer keys of the 128K decode shape (16 sequences x
    32768 entries x 128 dims, bf16 N(0,1) rows with per-row power-of-two spreads) in one call."""
    import torch
    from csa_synth import normal_kv, streams
    import long_context_compressed_03_amd as csa
    n, d = QUANT_SHAPE
    (r,) = streams(91, 0, 1)
    x = normal_kv(r, (n, d), "f32") * np.exp2(r.integers(-4, 5, (n, 1))).astype(np.float32)
    from csa_synth import f32_to_bf16_bits
    bits = f32_to_bf16_bits(x)
    st = Step(QUANT_WORKLOAD, n)
    nbytes = n * (2 * d + d // 2 + d // 32)

    def f_quant(c):
        csa.csa_mxfp4_quantize(c["x"], c["codes"], c["e8m0"])
    st.add(Kernel("mxfp4_quantize", f_quant, nbytes, 0, BF16_PEAK_TFLOPS, "mxfp4_quantize", "mxfp4_quantize_kernel"))
    R = args.rotate or max(2, math.ceil(600e6 / nbytes))
    base = {"x": torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda(),
            "codes": torch.empty((n, d // 2), dtype=torch.uint8, device="cuda"),
            "e8m0": torch.empty((n, d // 32), dtype=torch.uint8, device="cuda")}
    st.copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    st.layers = [("", {"quant_sample": bits[:8192]})]
    st.config = {"workload": QUANT_WORKLOAD, "vectors": n, "d": d, "input": "bf16",
                 "output": "MXFP4 (E2M1 codes + E8M0 per 32)"}
    return st


APPEND_WORKLOAD = "kv_append_decode_128k"
APPEND_SHAPE = dict(B=16, L=128, m=4, cap=32768, pos=131071)


def build_append(args):
    """One decode step's cache append for a CSA layer of the 128K decode shape: 16 sequences,
    each appending its token at position 131071, which completes a block of m = 4.  The K/V
    token goes to a 128-token bf16 window ring and the block is pooled into fp8 entry 32767;
    the token's indexer key goes to its own ring, is pooled into an fp32 entry, and that entry
    is converted to the indexer's MXFP4 key cache."""
    import torch
    from csa_synth import compress_inputs
    import long_context_compressed_03_amd as csa
    B, L, m, cap, p = (APPEND_SHAPE[k] for k in ("B", "L", "m", "cap", "pos"))
    x = compress_inputs(B, 2 * L + 1, "bf16", seed=17)
    xi = compress_inputs(B, 2 * L + 1, "bf16", seed=18)      # indexer keys
    st = Step(APPEND_WORKLOAD, B)
    # per sequence: the new K/V rows and logit read; 2 copies of each written; the block's
    # m K/V rows and logits read back; the fp8 entries and scales written; pos, plan, base
    nbytes = B * (2 * 256 + 4 + 2 * (2 * 256 + 4) + m * (2 * 256 + 4) + 2 * (128 + 4) + 4 + 8 + 8 + 4)

    # per sequence: the K/V token's rows and logit read, 2 copies written, the block's m K/V
    # rows and logits read back, the fp8 entries and scales written; the indexer key's row and
    # logit read, 2 copies written, its block's m rows and logits read back, the 64 + 4 B MXFP4
    # entry written; pos and the window base
    nbytes = B * ((2 * 256 + 4 + 2 * (2 * 256 + 4) + m * (2 * 256 + 4) + 2 * (128 + 4))
                  + (256 + 4 + 2 * (256 + 4) + m * (256 + 4) + 68) + 4 + 4)

    def f_append(c):
        csa.csa_decode_append(c["k_new"], c["v_new"], c["z_new"], c["ik_new"], c["z_new"], c["pos"], c["rk"],
                              c["rv"], c["rz"], m, c["ck"], c["cv"], c["irk"], c["rz_i"], c["kc"], c["ke"],
                              ck_scale=c["cks"], cv_scale=c["cvs"], raw_pos0=c["raw0"])
    st.add(Kernel("decode_append", f_append, nbytes, 0, BF16_PEAK_TFLOPS, "decode_append",
                  "decode_append_kernel"))
    K = torch.from_numpy(x["K"].view(np.int16)).view(torch.bfloat16).cuda()
    V = torch.from_numpy(x["V"].view(np.int16)).view(torch.bfloat16).cuda()
    Z = torch.from_numpy(x["logits"]).cuda()
    Vx = torch.from_numpy(xi["K"].view(np.int16)).view(torch.bfloat16).cuda()
    base = {"rk": K[:, :2 * L].contiguous(), "rv": V[:, :2 * L].contiguous(), "rz": Z[:, :2 * L].contiguous(),
            "k_new": K[:, 2 * L].contiguous(), "v_new": V[:, 2 * L].contiguous(),
            "z_new": Z[:, 2 * L].contiguous(),
            "pos": torch.full((B,), p, dtype=torch.int32, device="cuda"),
            "ck": torch.zeros((B, cap, 128), dtype=torch.uint8, device="cuda"),
            "cv": torch.zeros((B, cap, 128), dtype=torch.uint8, device="cuda"),
            "cks": torch.zeros((B, cap), device="cuda"), "cvs": torch.zeros((B, cap), device="cuda"),
            "raw0": torch.empty((B,), dtype=torch.int32, device="cuda"),
            # the indexer keys' ring (d_I = 128) and MXFP4 key cache
            "irk": Vx[:, :2 * L].contiguous(), "rz_i": Z[:, :2 * L].contiguous(),
            "ik_new": Vx[:, 2 * L].contiguous(),
            "kc": torch.zeros((B, cap, 64), dtype=torch.uint8, device="cuda"),
            "ke": torch.zeros((B, cap, 4), dtype=torch.uint8, device="cuda")}
    R = args.rotate or 4
    st.copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    st.layers = [("", {"append_sample": {k: x[k][:, :2 * L + 1] for k in ("K", "V", "logits")},
                        "append_sample_ix": xi["K"][:, :2 * L + 1]})]
    st.config = {"workload": APPEND_WORKLOAD, "batch": B, "position": p, "ring_tokens": L,
                 "block_m": m, "compressed_entries": cap, "window_kv": "bf16",
                 "compressed_kv": "fp8_e4m3+fp32 scale", "pooling": "every step (the block completes)",
                 "indexer_keys": "own ring, fp32 entries, MXFP4 (E2M1 + E8M0 per 32) key cache"}
    return st


def build(args):
    """Host inputs, R device copies and the step's launches for the chosen workload."""
    import torch
    if args.workload == QUANT_WORKLOAD:
        return build_quant(args)
    if args.workload == APPEND_WORKLOAD:
        return build_append(args)
    from csa_synth import workloads
    wls = workloads()
    if args.workload == "pair_1m":
        return build_pair(args, wls)
    parts = LAYERS[args.workload]
    hosts = [(prefix, host_layer(wls[name])) for prefix, name in parts]
    if args.workload == "pair_1m_split":
        q_tokens = wls["pair_csa_decode_1m"].B + wls["pair_csa_chunk_1m"].T_q
    else:
        q_tokens = hosts[0][1]["wl"].B * hosts[0][1]["wl"].T_q
    st = Step(args.workload, q_tokens)
    for prefix, h in hosts:
        add_layer(st, h, prefix, args.indexer, args.batch_invariant)
    per_copy = sum(k.nbytes for k in st.kernels.values())
    R = args.rotate or max(2, math.ceil(600e6 / per_copy))
    base = {}
    for prefix, h in hosts:
        base.update(device_layer(h, prefix))
    base = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
    st.copies = [base] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v)
                           for k, v in base.items()} for _ in range(R - 1)]
    st.layers = hosts
    if args.workload == "pair_1m_split":
        st.config = {"workload": args.workload, "layers": "CSA then HCA, same query tokens",
                     "step": "decode rows and the chunk in separate calls per op",
                     **{prefix.rstrip("."): layer_config(h["wl"]) for prefix, h in hosts}}
    else:
        st.config = {"workload": args.workload, **layer_config(hosts[0][1]["wl"])}
    st.config["indexer_topk"] = ("combined with the compression" if any(n.endswith("compress_indexer_topk") for n in st.order)
                                 else "fused" if any(n.endswith("indexer_topk") for n in st.order) else "unfused")
    if args.batch_invariant:
        st.config["attention"] = "batch-invariant calls"
    return st


def build_pair(args, wls):
    """The 1M layer pair's mixed step: 4 decode rows and one 2048-token chunk packed into one
    varlen call per op (compression, indexer top-k and sparse attention of the CSA layer;
    compression and dense attention of the HCA layer), all captured in one graph."""
    import torch
    hosts = [(prefix, host_layer(wls[name])) for prefix, name in LAYERS["pair_1m_split"]]
    hd = {prefix.rstrip("."): h for prefix, h in hosts}
    q_tokens = wls["pair_csa_decode_1m"].B + wls["pair_csa_chunk_1m"].T_q
    st = Step("pair_1m", q_tokens)
    base = {}
    for kind in ("csa", "hca"):
        dec, ch = hd[kind + "_decode"], hd[kind + "_chunk"]
        pk = pack_layer(dec, ch)
        add_varlen_layer(st, dec, ch, kind + ".")
        base.update(device_packed(pk, kind + ".", kind, dec["wl"].k))
        del pk
    per_copy = sum(k.nbytes for k in st.kernels.values())
    R = args.rotate or max(2, math.ceil(600e6 / per_copy))
    base = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
    st.copies = [base] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v)
                           for k, v in base.items()} for _ in range(R - 1)]
    st.layers = hosts
    st.config = {"workload": "pair_1m", "layers": "CSA then HCA, same query tokens",
                 "step": "4 decode rows + one 2048-token chunk packed into one call per op (varlen: "
                         "compress, indexer top-k, sparse attention; compress, dense attention)",
                 **{prefix.rstrip("."): layer_config(h["wl"]) for prefix, h in hosts}}
    st.config["indexer_topk"] = "fused, packed rows"
    st.config["attention"] = "varlen calls, plain plan (many-query kernel with split decode rows for HCA)"
    return st


# --------------------------------------------------------------------------
# Timing

def time_step(st, steps, warmup, use_graph, dist_steps):
    """Time exactly `steps` steps after `warmup` untimed ones.

    With graphs, the steps of all R input copies are captured into one graph, and
    the steps of the first `steps mod R` copies into a second; the timed region
    replays the first floor(steps / R) times and the second once, so exactly
    `steps` steps run back to back between the two events, every copy in turn.
    The distribution comes from `dist_steps` further replays of the R-step graph,
    each between its own pair of events: per replay, the mean step time over
    its R steps.  Returns (ms per step, steps, wall seconds, per-step stats)."""
    import torch
    R = len(st.copies)
    for i in range(warmup):
        st.run(st.copies[i % R])
    torch.cuda.synchronize()
    n_full, rem = divmod(steps, R)
    full = part = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in st.copies:      # one eager pass on the capture stream first
                st.run(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(full):
            for c in st.copies:
                st.run(c)
        if rem:
            part = torch.cuda.CUDAGraph()
            with torch.cuda.graph(part):
                for c in st.copies[:rem]:
                    st.run(c)
        torch.cuda.synchronize()
        full.replay()
        if part is not None:
            part.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    if use_graph:
        for _ in range(n_full):
            full.replay()
        if part is not None:
            part.replay()
    else:
        for i in range(steps):
            st.run(st.copies[i % R])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    n = max(dist_steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        if use_graph:
            full.replay()
        else:
            for c in st.copies:
                st.run(c)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / R for a, b in ev])
    stats = {"replays": n, "steps_per_replay": R, "median_us": round(float(np.median(us)), 3),
             "p10_us": round(float(np.percentile(us, 10)), 3), "p90_us": round(float(np.percentile(us, 90)), 3),
             "how": "mean step time of each replay of the all-copies step graph, each replay between its own "
                    "pair of HIP events" if use_graph else "mean step time of each eager pass over the copies"}
    del full, part
    return ms / steps, steps, wall, stats


def time_kernels(st, reps):
    """Average duration of each call, from HIP events on its stream.

    Each call is captured alone, once per input copy, into a HIP graph; the
    graph is replayed and bracketed by events, so the figure is device time per
    call (back-to-back launches, no host gap) over the rotating inputs.
    """
    import torch
    R = len(st.copies)
    res = {}
    for name in st.order:
        fn = st.kernels[name].fn
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in st.copies:
                fn(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for c in st.copies:
                fn(c)
        gr.replay()
        torch.cuda.synchronize()
        n_rep = max(1, reps // R)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_rep):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (n_rep * R)
        res[name] = {"avg_us": us, "launches": n_rep * R}
        del gr
    # restore the step's data flow (each call above ran on the previous call's outputs)
    for c in st.copies:
        st.run(c)
    torch.cuda.synchronize()
    return res


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "long_context_compressed_03_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "indexer_scores": ["indexer.hip", "indexer_core.hpp", "select.hpp", "common.hpp"],
    "indexer_topk": ["indexer_topk.hip", "indexer_core.hpp", "split.hpp", "topk.hip", "select.hpp",
                     "compress_core.hpp", "common.hpp"],
    "sparse_attn": ["attn.hip", "common.hpp"], "dense_attn": ["attn.hip", "common.hpp"],
    "topk": ["topk.hip", "split.hpp", "select.hpp", "compress_core.hpp", "common.hpp"],
    "compress_kv": ["compress.hip", "compress_core.hpp", "common.hpp"],
    "compress_indexer_topk": ["indexer_topk.hip", "indexer_core.hpp", "split.hpp", "topk.hip", "select.hpp",
                              "compress_core.hpp", "compress.hip", "common.hpp"],
    "mxfp4_quantize": ["quant.hip", "mxfp4.hpp", "common.hpp"],
    "kv_cache_append": ["cache.hip", "compress.hip", "compress_core.hpp", "mxfp4.hpp", "common.hpp"],
    "indexer_key_append": ["cache.hip", "compress_core.hpp", "mxfp4.hpp", "common.hpp"],
    "decode_append": ["cache.hip", "compress_core.hpp", "mxfp4.hpp", "common.hpp"]}


def measured_traffic(workload, kernel):
    """HBM bytes per call from a committed rocprofv3 counter summary, if still current.

    The summary (profiles/<call>_<workload>_pmc.json) holds FETCH_SIZE + WRITE_SIZE
    per call, scaled by what the same counters read for a plain 256 MiB device copy,
    and the hash of the call's kernel sources when it was taken; a changed kernel
    gives null.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel.name.replace('.', '_')}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel.src]):
        return None
    return d.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload

def cpu_baseline_quant(st):
    """The oracle's MXFP4 encoder on 8192 of the workload's vectors, in vectors/s."""
    from oracle.formats import bf16_decode, mxfp4_encode
    sample = st.layers[0][1]["quant_sample"]
    x = bf16_decode(sample)
    t0 = time.perf_counter()
    mxfp4_encode(x)
    dt = time.perf_counter() - t0
    return len(sample) / dt, f"fp64 numpy oracle encoder on {len(sample)} of the workload's vectors ({dt:.2f} s)"


def cpu_baseline_append(st, budget_s=10.0):
    """The oracle's cache append (ring writes as the step-by-step definition states them,
    the pool of the completed block, and the same for the indexer key with its MXFP4
    encoding) for the workload's 16 sequences, repeated within the budget; appended
    tokens/s."""
    from oracle.cache import append_step_by_step
    from oracle.compress import compress_kv
    from oracle.formats import bf16_decode, mxfp4_encode
    x = st.layers[0][1]["append_sample"]
    L, m, p = APPEND_SHAPE["L"], APPEND_SHAPE["m"], APPEND_SHAPE["pos"]
    K, V, Z = bf16_decode(x["K"]), bf16_decode(x["V"]), x["logits"]
    KI = bf16_decode(st.layers[0][1]["append_sample_ix"])
    B = K.shape[0]
    reps, t0 = 0, time.perf_counter()
    while True:
        for b in range(B):
            for X in (K[b], V[b], Z[b], KI[b]):
                append_step_by_step(X, X.shape[0], L, start=X.shape[0] - 1)   # the newest token
            compress_kv(K[b:b + 1, -m:], V[b:b + 1, -m:], Z[b:b + 1, -m:], m, "fp8")
            ik, _ = compress_kv(KI[b:b + 1, -m:], KI[b:b + 1, -m:], Z[b:b + 1, -m:], m, "f32")
            mxfp4_encode(ik.astype(np.float64))
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return reps * B / dt, (f"fp64 numpy oracle: {reps} appends of the workload's {B} tokens at "
                           f"position {p} (ring writes, fp8 pooling of the completed block, the indexer "
                           f"key's ring, fp32 pool and MXFP4 encoding), {dt:.1f} s")


def cpu_baseline(st, budget_s):
    """The oracle, timed on the host on a sample of the step's query rows.

    Per layer: the compression of the step's pooled rows and the decoding of the
    stored caches of one sequence are timed once; indexer, top-k and attention are
    timed per sampled query row (decode layers: one row per sequence, chunk layers:
    rows spread evenly over the chunk).  The step's oracle time is the fixed part
    plus the mean row time times the step's rows, per layer.  BLAS runs one
    thread per host core it may run on (os.sched_getaffinity).  Returns
    (query-tokens/s, description, threads).
    """
    from threadpoolctl import threadpool_limits
    import oracle.attention as oa
    import oracle.compress as oc
    import oracle.indexer as oi
    import oracle.topk as ot
    from oracle.formats import bf16_decode
    total, parts = 0.0, []
    share = budget_s / len(st.layers)
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        for prefix, h in st.layers:
            wl, kv, at, ix = h["wl"], h["kv"], h["at"], h.get("ix")
            L, row0, _ = pool_range(wl)
            sl = slice(row0, row0 + L)
            t0 = time.perf_counter()
            Kw, Vw = bf16_decode(kv["K"][:, sl]), bf16_decode(kv["V"][:, sl])
            oc.compress_kv(Kw, Vw, kv["logits"][:, sl], wl.m, wl.ckv)
            t_fixed = time.perf_counter() - t0

            def seq_arrays(b):
                cK = oa.decode_kv(at["cK"][b:b + 1], wl.ckv,
                                  None if at["cK_scale"] is None else at["cK_scale"][b:b + 1])
                cV = oa.decode_kv(at["cV"][b:b + 1], wl.ckv,
                                  None if at["cV_scale"] is None else at["cV_scale"][b:b + 1])
                return cK, cV, bf16_decode(kv["K"][b:b + 1]), bf16_decode(kv["V"][b:b + 1])
            if wl.T_q == 1:
                rows = [(b, 0) for b in range(wl.B)]
                cached = None
            else:
                n_s = 64
                rows = [(0, int(i)) for i in np.linspace(0, wl.T_q - 1, n_s).round()]
                t0 = time.perf_counter()
                cached = seq_arrays(0)
                t_fixed += time.perf_counter() - t0
            t_rows = []
            t_layer0 = time.perf_counter()
            for b, i in rows:
                if t_rows and sum(t_rows) > share:
                    break
                t = wl.q_pos0[b] + i
                pos = np.array([t])
                r0 = np.array([wl.raw_pos0[b]])
                t0 = time.perf_counter()
                cK, cV, Kb, Vb = cached if cached is not None else seq_arrays(b)
                q = bf16_decode(at["q"][b:b + 1, i:i + 1])
                if wl.kind == "csa":
                    s = oi.indexer_scores(ix["q_codes"][b:b + 1, i:i + 1],
                                          ix["q_e8m0"][b:b + 1, i:i + 1], ix["w"][b:b + 1, i:i + 1],
                                          ix["k_codes"][b:b + 1], ix["k_e8m0"][b:b + 1], pos, wl.m)
                    idx = ot.topk(s.astype(np.float32), pos, wl.m, wl.k)
                    oa.sparse_attn(q, cK, cV, idx, Kb, Vb, r0, pos, wl.W)
                else:
                    oa.dense_attn(q, cK, cV, wl.m, Kb, Vb, r0, pos, wl.W)
                t_rows.append(time.perf_counter() - t0)
                if time.perf_counter() - t_layer0 > 3 * share:
                    break
            n_step_rows = wl.B * wl.T_q
            total += t_fixed + n_step_rows * float(np.mean(t_rows))
            parts.append(f"{prefix.rstrip('.') or wl.name}: {len(t_rows)} of {n_step_rows} query rows "
                         f"({sum(t_rows):.1f} s) + pooling of the step's blocks")
    desc = ("fp64 numpy oracle (compress, indexer, top-k, attention) on a sample of the same "
            f"workload's query rows, scaled to one step, BLAS on {cores} threads (its einsum "
            "reductions run on one); " + "; ".join(parts))
    return st.q_tokens / total, desc, cores


def hip_kernels(st, name):
    """The HIP kernels a call of this step launches, by the shapes the library dispatches on
    (for matching the call's event time against rocprofv3 kernel traces)."""
    return st.kernels[name].hip


def roofline_entry(k, avg_us):
    s = avg_us * 1e-6
    if k.bound == "hbm":
        return k.nbytes / s / 1e9, HBM_PEAK_GBS, "GB/s"
    return k.flops / s / 1e12, k.mfma_peak, "TFLOP/s"


SUB_WORKLOADS = ["csa_decode_128k", "hca_decode_1m", "csa_prefill_256k", "pair_1m_split"]
HEADLINE = "pair_1m"


def measure(args, workload, with_cpu):
    """Build one workload, time it (exact steps, distribution, each call) and return its
    figures as a dict; the device copies are freed before returning."""
    import torch
    args.workload = workload
    st = build(args)
    ms, done, wall, stats = time_step(st, args.steps, args.warmup, not args.no_graph, args.dist_steps)
    kt = time_kernels(st, reps=max(10 * len(st.copies), 200))
    # dominant call = largest share of the step
    dom = max(st.order, key=lambda n: kt[n]["avg_us"])
    k = st.kernels[dom]
    achieved, peak, unit = roofline_entry(k, kt[dom]["avg_us"])
    roof = {"kernel": dom, "hip_kernels": hip_kernels(st, dom), "bound": k.bound, "achieved": round(achieved, 1),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(workload, k),
            "algorithmic_bytes_per_launch": k.nbytes, "algorithmic_flops_per_launch": k.flops,
            "avg_launch_us": round(kt[dom]["avg_us"], 3)}
    kernels = {}
    for n in st.order:
        kk = st.kernels[n]
        a_, p_, u_ = roofline_entry(kk, kt[n]["avg_us"])
        kernels[n] = {"avg_us": round(kt[n]["avg_us"], 3), "hip_kernels": hip_kernels(st, n),
                      "algorithmic_bytes": kk.nbytes, "algorithmic_flops": kk.flops, "bound": kk.bound,
                      "achieved": round(a_, 1), "unit": u_, "frac": round(a_ / p_, 4)}
    quant = workload == QUANT_WORKLOAD
    append = workload == APPEND_WORKLOAD
    unit_v = "key-vectors/s" if quant else "appended-tokens/s" if append else "query-tokens/s"
    cpu = None
    if with_cpu:
        cores = 1
        if quant:
            v, desc = cpu_baseline_quant(st)
        elif append:
            v, desc = cpu_baseline_append(st, args.cpu_seconds)
        else:
            v, desc, cores = cpu_baseline(st, args.cpu_seconds)
        cpu = {"value": round(v, 4), "unit": unit_v, "cores": cores, "kind": "oracle", "sample": desc}
    res = {"value": round(st.q_tokens / (ms * 1e-3), 1), "unit": unit_v, "steps": done,
           "ms_per_step": round(ms, 5), "step_stats": stats, "config": st.config, "roofline": roof,
           "cpu_baseline": cpu, "kernels": kernels,
           ("vectors_per_step" if quant else "tokens_per_step" if append else "query_tokens_per_step"): st.q_tokens,
           "rotation_copies": len(st.copies), "graph": not args.no_graph, "wall_s_timed_region": round(wall, 4)}
    st.copies = []
    del st
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding is a "
                                   "design (context-sharded top-k + LSE combine), not measured",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    import long_context_compressed_03_amd as csa
    csa.load()
    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        c = torch.empty_like(a)
        for _ in range(10):
            c.copy_(a)
        torch.cuda.synchronize()
        del a, c
    with_cpu = not args.no_cpu_baseline
    subs = {}
    if args.workload == "all":
        for w in SUB_WORKLOADS:
            print(f"# {w}", file=sys.stderr, flush=True)
            subs[w] = measure(args, w, False)
        print(f"# {HEADLINE}", file=sys.stderr, flush=True)
        head, name = measure(args, HEADLINE, with_cpu), HEADLINE
    else:
        name = args.workload
        head = measure(args, name, with_cpu)
    metric = ("MXFP4 quantisation of the indexer keys, key-vectors/s; % HBM roofline" if name == QUANT_WORKLOAD else
              "decode KV cache append (window ring + block pooling), appended tokens/s" if name == APPEND_WORKLOAD
              else METRIC)
    line = {"metric": metric, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
            "steps": head["steps"], "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "mxfp4+bf16", "data": "synthetic (seeded; shapes of the pages' 128K-1M contexts)",
            "config": head["config"], "roofline": head["roofline"], "cpu_baseline": head["cpu_baseline"]}
    line.update({k: v for k, v in head.items() if k not in line and k not in ("value", "unit")})
    if subs:
        line["workloads"] = subs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
