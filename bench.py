"""Benchmark of the CSA / HCA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input.  The
default workload is CSA decoding at a 128K context: 16 sequences, one query
each at position 131071; the block of 4 tokens the query completes is pooled
into compressed entry 32767, the MXFP4 indexer scores all 32768 entries (8
heads x 128), the top 1024 are kept and 64-head attention runs over them plus
the 128-token window.  Other workloads (--workload) cover HCA decoding at 1M,
CSA prefill of a 4096-token chunk at 256K, and the 1M CSA+HCA layer pair.

Inputs are resident in HBM before timing.  The step is captured once per input
copy into a HIP graph; copies rotate so that one rotation touches well over
twice the 256 MB Infinity Cache and reads are served by HBM.  Per-kernel
durations come from HIP events around eager launches of each kernel on the
stream it runs on.  The CPU oracle is timed on a bounded sample of the same
workload on the host.

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
    p.add_argument("--steps", type=int, default=240)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="csa_decode_128k",
                   choices=["csa_decode_128k", "hca_decode_1m", "csa_prefill_256k", "pair_1m"])
    p.add_argument("--rotate", type=int, default=0, help="input copies (0 = auto)")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run 10 plain device copies of 256 MiB (reference for HBM byte counters)")
    return p.parse_args()


# --------------------------------------------------------------------------
# Workload construction (device tensors)

class Step:
    """One workload: device inputs (R rotating copies) and the launches of one step."""

    def __init__(self, name, q_tokens):
        self.name = name
        self.q_tokens = q_tokens
        self.copies = []
        self.kernels = {}     # name -> (fn(copy), algorithmic bytes, flops, bound)
        self.order = []
        self.config = {}

    def add(self, name, fn, nbytes, flops, bound):
        self.kernels[name] = (fn, nbytes, flops, bound)
        self.order.append(name)

    def run(self, c):
        for n in self.order:
            self.kernels[n][0](c)


def _dev_copies(tensors, R):
    import torch
    base = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in tensors.items()}
    out = [base]
    for _ in range(R - 1):
        out.append({k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in base.items()})
    return out


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


def csa_decode_tensors(wl, seed=0):
    """Host inputs of a CSA decode step (wl: csa_synth Workload)."""
    import torch
    from csa_synth import attn_inputs, compress_inputs, indexer_inputs
    B, cap, W, H = wl.B, wl.cap, wl.W, wl.H
    kv = compress_inputs(B, wl.L_raw, "bf16", seed=seed, tag=wl.tag * 10 + 1, outliers=wl.outliers)
    ix = indexer_inputs(B, 1, cap, wl.H_I, wl.d_I, seed=seed, tag=wl.tag * 10 + 2)
    at = attn_inputs(B, 1, H, cap, 1, "bf16", wl.ckv, seed=seed, tag=wl.tag * 10 + 3,
                     outliers=wl.outliers)
    T = dict(kw=_t(kv["K"], "bf16"), vw=_t(kv["V"], "bf16"), logits=_t(kv["logits"], "f32"),
             qc=_t(ix["q_codes"], "u8"), qe=_t(ix["q_e8m0"], "u8"), w=_t(ix["w"], "f32"),
             kc=_t(ix["k_codes"], "u8"), ke=_t(ix["k_e8m0"], "u8"), q=_t(at["q"], "bf16"),
             pos=_t(np.array(wl.q_pos0), "i32"), raw0=_t(np.array(wl.raw_pos0), "i32"))
    if wl.ckv == "fp8":
        T.update(ck=_t(at["cK"], "u8"), cv=_t(at["cV"], "u8"), cks=_t(at["cK_scale"], "f32"),
                 cvs=_t(at["cV_scale"], "f32"))
    else:
        T.update(ck=_t(at["cK"], "bf16"), cv=_t(at["cV"], "bf16"), cks=None, cvs=None)
    T["scores"] = torch.empty((B, 1, cap), dtype=torch.float32)
    T["idx"] = torch.empty((B, 1, wl.k), dtype=torch.int32)
    T["out"] = torch.empty((B, 1, H, 128), dtype=torch.bfloat16)
    return T


def build_csa_decode(wl, R):
    import long_context_compressed_03_amd as csa
    T = csa_decode_tensors(wl)
    copies = _dev_copies(T, R)
    B, cap, m, k, W, H = wl.B, wl.cap, wl.m, wl.k, wl.W, wl.H
    st = Step(wl.name, B)
    st.copies = copies
    ent = 264 if wl.ckv == "fp8" else 512
    idx_bytes = wl.d_I // 2 + wl.d_I // 32

    def f_compress(c):
        csa.csa_compress_kv(c["kw"], c["vw"], c["logits"], m, c["ck"], c["cv"], c["cks"], c["cvs"],
                            L=m, row0=wl.L_raw - m, entry0=cap - 1)

    def f_indexer(c):
        csa.csa_indexer_scores(c["qc"], c["qe"], c["w"], c["kc"], c["ke"], c["pos"], m, c["scores"])

    def f_topk(c):
        csa.csa_topk(c["scores"], c["pos"], m, k, c["idx"])

    def f_attn(c):
        csa.csa_sparse_attn(c["q"], c["ck"], c["cv"], c["idx"], c["kw"], c["vw"], c["raw0"], c["pos"],
                            W, ck_scale=c["cks"], cv_scale=c["cvs"], out=c["out"])
    st.add("compress_kv", f_compress, B * (m * 512 + m * 4 + ent), 0, "hbm")
    st.add("indexer_scores", f_indexer, B * cap * (idx_bytes + 4), 2 * B * cap * wl.H_I * wl.d_I,
           "hbm")
    st.add("topk", f_topk, B * cap * 4 + B * k * 4, 0, "hbm")
    st.add("sparse_attn", f_attn, B * (k * ent + W * 512 + H * 128 * 4), 4 * B * H * 128 * (k + W),
           "hbm")
    st.config = {"workload": wl.name, "batch": B, "context": wl.q_pos0[0] + 1, "query_heads": H,
                 "kv_heads": 1, "head_dim": 128, "m": m, "compressed_entries": cap,
                 "indexer": f"{wl.H_I}x{wl.d_I} MXFP4", "top_k": k, "window": W,
                 "compressed_kv": wl.ckv, "window_kv": "bf16"}
    return st


def build_hca_decode(wl, R):
    import torch
    import long_context_compressed_03_amd as csa
    from csa_synth import attn_inputs, compress_inputs
    B, cap, mp, W, H = wl.B, wl.cap, wl.m, wl.W, wl.H
    kv = compress_inputs(B, wl.L_raw, "bf16", seed=0, tag=wl.tag * 10 + 1, outliers=wl.outliers)
    at = attn_inputs(B, 1, H, cap, 1, "bf16", "fp8", seed=0, tag=wl.tag * 10 + 3,
                     outliers=wl.outliers)
    T = dict(kw=_t(kv["K"], "bf16"), vw=_t(kv["V"], "bf16"), logits=_t(kv["logits"], "f32"),
             q=_t(at["q"], "bf16"), ck=_t(at["cK"], "u8"), cv=_t(at["cV"], "u8"),
             cks=_t(at["cK_scale"], "f32"), cvs=_t(at["cV_scale"], "f32"),
             pos=_t(np.array(wl.q_pos0), "i32"), raw0=_t(np.array(wl.raw_pos0), "i32"),
             out=torch.empty((B, 1, H, 128), dtype=torch.bfloat16))
    st = Step(wl.name, B)
    st.copies = _dev_copies(T, R)

    def f_compress(c):
        csa.csa_compress_kv(c["kw"], c["vw"], c["logits"], mp, c["ck"], c["cv"], c["cks"], c["cvs"],
                            L=mp, row0=wl.L_raw - mp, entry0=cap - 1)

    def f_attn(c):
        csa.hca_dense_attn(c["q"], c["ck"], c["cv"], mp, c["kw"], c["vw"], c["raw0"], c["pos"], W,
                           ck_scale=c["cks"], cv_scale=c["cvs"], out=c["out"])
    st.add("compress_kv", f_compress, B * (mp * 516 + 264), 0, "hbm")
    st.add("dense_attn", f_attn, B * (cap * 264 + W * 512 + H * 128 * 4), 4 * B * H * 128 * (cap + W),
           "hbm")
    st.config = {"workload": wl.name, "batch": B, "context": wl.q_pos0[0] + 1, "query_heads": H,
                 "kv_heads": 1, "head_dim": 128, "m_prime": mp, "compressed_entries": cap,
                 "window": W, "compressed_kv": "fp8_e4m3+fp32 scale", "window_kv": "bf16"}
    return st


def build(args):
    from csa_synth import workloads
    wls = workloads()
    if args.workload == "csa_decode_128k":
        wl = wls["csa_decode_128k"]
        per_copy = wl.B * wl.cap * (68 + 4) + wl.B * wl.k * 512 + wl.B * 128 * 512
        R = args.rotate or max(2, math.ceil(600e6 / per_copy))
        return build_csa_decode(wl, R)
    if args.workload == "hca_decode_1m":
        wl = wls["hca_decode_1m"]
        per_copy = wl.B * wl.cap * 264
        R = args.rotate or max(2, math.ceil(600e6 / per_copy))
        return build_hca_decode(wl, R)
    raise SystemExit(f"workload {args.workload} is not wired into the benchmark yet")


# --------------------------------------------------------------------------
# Timing

def time_step(st, steps, warmup, use_graph):
    import torch
    R = len(st.copies)
    for i in range(warmup):
        st.run(st.copies[i % R])
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in st.copies:      # one eager pass on the capture stream first
                st.run(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in st.copies:
                st.run(c)
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    n_rep = max(1, steps // R) if use_graph else steps
    done = n_rep * R if use_graph else steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    if use_graph:
        for _ in range(n_rep):
            graph.replay()
    else:
        for i in range(steps):
            st.run(st.copies[i % R])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    return ms / done, done, wall


def time_kernels(st, reps):
    """Average duration of each kernel, from HIP events on its stream.

    Each kernel is captured alone, once per input copy, into a HIP graph; the
    graph is replayed and bracketed by events, so the figure is device time per
    launch (back-to-back launches, no host gap) over the rotating inputs.
    """
    import torch
    R = len(st.copies)
    res = {}
    for name in st.order:
        fn = st.kernels[name][0]
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
    # restore the step's data flow (each kernel above ran on the previous kernel's outputs)
    for c in st.copies:
        st.run(c)
    torch.cuda.synchronize()
    return res


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "long_context_compressed_03_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"indexer_scores": ["indexer.hip", "common.hpp"],
                  "sparse_attn": ["attn.hip", "common.hpp"], "dense_attn": ["attn.hip", "common.hpp"],
                  "topk": ["topk.hip", "common.hpp"], "compress_kv": ["compress.hip", "common.hpp"]}


def measured_traffic(workload, kernel):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if still current.

    The summary (profiles/<kernel>_<workload>_pmc.json) holds FETCH_SIZE + WRITE_SIZE
    per dispatch of the kernel, scaled by what the same counters read for a plain
    256 MiB device copy, and the hash of the kernel's sources when it was taken; a
    changed kernel gives null.
    """
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload

def cpu_baseline_timed(workload, budget_s):
    """Time only the oracle's arithmetic (input generation and decoding excluded)."""
    from csa_synth import attn_inputs, compress_inputs, indexer_inputs, workloads
    import oracle.attention as oa
    import oracle.compress as oc
    import oracle.indexer as oi
    import oracle.topk as ot
    from oracle.formats import bf16_decode
    wl = workloads()[workload]
    done, spent, seed = 0, 0.0, 0
    wall0 = time.perf_counter()
    while spent < budget_s and time.perf_counter() - wall0 < 3 * budget_s:
        kv = compress_inputs(1, wl.L_raw, "bf16", seed=seed, tag=wl.tag * 10 + 1)
        at = attn_inputs(1, 1, wl.H, wl.cap, 1, "bf16", wl.ckv, seed=seed, tag=wl.tag * 10 + 3)
        ix = (indexer_inputs(1, 1, wl.cap, wl.H_I, wl.d_I, seed=seed, tag=wl.tag * 10 + 2)
              if wl.kind == "csa" else None)
        pos = np.array(wl.q_pos0[:1])
        raw0 = np.array(wl.raw_pos0[:1])
        t0 = time.perf_counter()
        Kw, Vw = bf16_decode(kv["K"]), bf16_decode(kv["V"])
        oc.compress_kv(Kw[:, -wl.m:], Vw[:, -wl.m:], kv["logits"][:, -wl.m:], wl.m, wl.ckv)
        cK = oa.decode_kv(at["cK"], wl.ckv, at["cK_scale"])
        cV = oa.decode_kv(at["cV"], wl.ckv, at["cV_scale"])
        q = bf16_decode(at["q"])
        if wl.kind == "csa":
            s = oi.indexer_scores(ix["q_codes"], ix["q_e8m0"], ix["w"], ix["k_codes"], ix["k_e8m0"],
                                  pos, wl.m)
            idx = ot.topk(s.astype(np.float32), pos, wl.m, wl.k)
            oa.sparse_attn(q, cK, cV, idx, Kw, Vw, raw0, pos, wl.W)
        else:
            oa.dense_attn(q, cK, cV, wl.m, Kw, Vw, raw0, pos, wl.W)
        spent += time.perf_counter() - t0
        done += 1
        seed += 1
    return done, spent


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
    st = build(args)
    ms, done, wall = time_step(st, args.steps, args.warmup, not args.no_graph)
    kt = time_kernels(st, reps=max(10 * len(st.copies), 200))
    # dominant kernel = largest share of the step
    dom = max(st.order, key=lambda n: kt[n]["avg_us"])
    _, nbytes, flops, bound = st.kernels[dom]
    avg_s = kt[dom]["avg_us"] * 1e-6
    achieved = nbytes / avg_s / 1e9
    roof = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload, dom),
            "algorithmic_bytes_per_launch": int(nbytes), "avg_launch_us": round(kt[dom]["avg_us"], 3)}
    kernels = {}
    for n in st.order:
        _, b_, f_, _ = st.kernels[n]
        kernels[n] = {"avg_us": round(kt[n]["avg_us"], 3), "algorithmic_bytes": int(b_),
                      "GBps": round(b_ / (kt[n]["avg_us"] * 1e-6) / 1e9, 1)}
    cpu = None
    if not args.no_cpu_baseline:
        n_done, spent = cpu_baseline_timed(args.workload if args.workload != "pair_1m" else
                                           "csa_decode_128k", args.cpu_seconds)
        cpu = {"value": round(n_done / spent, 3), "unit": "query-tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n_done} single-sequence decode steps of the same workload at full "
                         f"context (fp64 numpy oracle; compress, indexer, top-k, attention), "
                         f"{spent:.1f} s of oracle arithmetic; input generation excluded"}
    q_per_s = st.q_tokens / (ms * 1e-3)
    line = {"metric": METRIC, "value": round(q_per_s, 1), "unit": "query-tokens/s", "n_gpus": 1,
            "steps": done, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "mxfp4+bf16", "data": "synthetic (seeded; shapes of the pages' 128K-1M contexts)",
            "config": st.config, "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
            "rotation_copies": len(st.copies), "graph": not args.no_graph,
            "wall_s_timed_region": round(wall, 4)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
