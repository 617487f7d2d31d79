"""Sampled parity at the full workload sizes, in the launch configuration the benchmark times.

Each test builds one workload exactly as bench.py does (same seeded inputs, same calls,
same order, same shapes), runs one step, and checks sampled outputs against the oracle,
which can afford a few rows at these sizes:
  * pooled entries written by the step: within one storage unit of the exact pool;
  * indexer scores of sampled rows (decode with separate indexer and top-k calls): bit-exact;
  * top-k indices of sampled rows (unfused, fused, and combined with the compression): bit-exact;
  * attention of sampled rows over the cache as the step left it: max-abs 2e-2 on top of
    the bf16 output's own half-unit rounding.
The 1M layer pair is checked layer by layer the same way, both as the packed mixed step
(one varlen call per op) and as separate calls per part.
"""
import numpy as np
import pytest
import torch

import bench
from csa_synth import workloads
from gpu_helpers import attention_tolerance, compress_tolerance, h, h_bf16, say
from oracle.attention import dense_attn, sparse_attn
from oracle.compress import compress_values, store
from oracle.formats import bf16_decode, e4m3_decode
from oracle.indexer import indexer_scores
from oracle.topk import topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def run_workload(name, indexer="auto"):
    """Host inputs and the device state after one step of bench workload `name`."""
    parts = bench.LAYERS[name]
    wls = workloads()
    hosts = [(prefix, bench.host_layer(wls[w])) for prefix, w in parts]
    st = bench.Step(name, 0)
    for prefix, hl in hosts:
        bench.add_layer(st, hl, prefix, indexer=indexer)
    dev = {}
    for prefix, hl in hosts:
        dev.update(bench.device_layer(hl, prefix))
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    say(f"{name}: calls {st.order}")
    st.run(dev)
    torch.cuda.synchronize()
    return hosts, dev, st


def cache_rows(dev, p, wl, b):
    """Compressed K/V of sequence b as the step left them (float64)."""
    if wl.ckv == "fp8":
        ks, vs = h(dev[p + "cks"])[b], h(dev[p + "cvs"])[b]
        return (e4m3_decode(h(dev[p + "ck"])[b]) * ks[:, None].astype(np.float64),
                e4m3_decode(h(dev[p + "cv"])[b]) * vs[:, None].astype(np.float64))
    return bf16_decode(h_bf16(dev[p + "ck"])[b]), bf16_decode(h_bf16(dev[p + "cv"])[b])


def check_compress(hl, dev, p, sample_entries):
    """Pooled entries the step wrote, against the exact pool of the same raw rows."""
    wl, kv = hl["wl"], hl["kv"]
    L, row0, entry0 = bench.pool_range(wl)
    m = wl.m
    for b in range(wl.B):
        K = bf16_decode(kv["K"][b, row0:row0 + L])
        V = bf16_decode(kv["V"][b, row0:row0 + L])
        z = kv["logits"][b, row0:row0 + L]
        for e in sample_entries:
            blk = slice(e * m, (e + 1) * m)
            Kh, Vh = compress_values(K[None, blk], V[None, blk], z[None, blk], m)
            for which, X, key in ((0, Kh[0, 0], "ck"), (1, Vh[0, 0], "cv")):
                amax = np.abs((K if which == 0 else V)[blk]).max()
                eps = (m + 4) * 2.0 ** -24 * amax
                if wl.ckv == "fp8":
                    codes, sc = store(X[None], "fp8")
                    o = e4m3_decode(codes[0]) * np.float64(sc[0])
                    g_sc = np.float64(h(dev[p + key + "s"])[b, entry0 + e])
                    assert abs(g_sc - sc[0]) <= eps / 448 + 2.0 ** -22 * sc[0]
                    g = e4m3_decode(h(dev[p + key])[b, entry0 + e]) * g_sc
                    tol = compress_tolerance(X[None], "fp8", eps, np.array([sc[0]]))[0]
                else:
                    o = bf16_decode(store(X, "bf16"))
                    g = bf16_decode(h_bf16(dev[p + key])[b, entry0 + e])
                    tol = compress_tolerance(X, "bf16", eps)
                assert np.all(np.abs(g - o) <= tol), f"entry {entry0 + e} of sequence {b}"


def row_scores(hl, b, i):
    wl, ix = hl["wl"], hl["ix"]
    pos = np.array([wl.q_pos0[b] + i])
    return indexer_scores(ix["q_codes"][b:b + 1, i:i + 1], ix["q_e8m0"][b:b + 1, i:i + 1],
                          ix["w"][b:b + 1, i:i + 1], ix["k_codes"][b:b + 1], ix["k_e8m0"][b:b + 1],
                          pos, wl.m)


def check_csa_rows(hl, dev, p, rows, unfused):
    wl, at, kv = hl["wl"], hl["at"], hl["kv"]
    g_idx = h(dev[p + "idx"])
    g_out = bf16_decode(h_bf16(dev[p + "out"]))
    g_scores = h(dev[p + "scores"]) if unfused else None
    Kw_all, Vw_all = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    for b, i in rows:
        t = wl.q_pos0[b] + i
        s = row_scores(hl, b, i)
        if unfused:
            assert np.array_equal(g_scores[b, i].astype(np.float64), s[0, 0]), f"scores row {(b, i)}"
        ref_idx = topk(s.astype(np.float32), np.array([t]), wl.m, wl.k)
        assert np.array_equal(g_idx[b, i], ref_idx[0, 0]), f"top-k row {(b, i)}"
        cK, cV = cache_rows(dev, p, wl, b)
        q = bf16_decode(at["q"][b:b + 1, i:i + 1])
        O, _ = sparse_attn(q, cK[None], cV[None], ref_idx, Kw_all[b:b + 1], Vw_all[b:b + 1],
                           np.array([wl.raw_pos0[b]]), np.array([t]), wl.W)
        diff = np.abs(g_out[b, i] - O[0, 0])
        say(f"  row {(b, i)}: top-k exact, attention err {diff.max():.2e}")
        assert np.all(diff <= attention_tolerance(O[0, 0], "bf16"))


def check_hca_rows(hl, dev, p, rows):
    wl, at, kv = hl["wl"], hl["at"], hl["kv"]
    g_out = bf16_decode(h_bf16(dev[p + "out"]))
    Kw_all, Vw_all = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    for b, i in rows:
        t = wl.q_pos0[b] + i
        cK, cV = cache_rows(dev, p, wl, b)
        q = bf16_decode(at["q"][b:b + 1, i:i + 1])
        O, _ = dense_attn(q, cK[None], cV[None], wl.m, Kw_all[b:b + 1], Vw_all[b:b + 1],
                          np.array([wl.raw_pos0[b]]), np.array([t]), wl.W)
        diff = np.abs(g_out[b, i] - O[0, 0])
        say(f"  row {(b, i)}: attention err {diff.max():.2e}")
        assert np.all(diff <= attention_tolerance(O[0, 0], "bf16"))


@pytest.mark.parametrize("indexer,call", [("auto", "compress_indexer_topk"), ("fused", "indexer_topk")])
def test_csa_decode_128k(csa, indexer, call):
    hosts, dev, st = run_workload("csa_decode_128k", indexer=indexer)
    (p, hl), = hosts
    assert call in st.order
    say(f"csa_decode_128k ({call}): pooled entry, fused top-k and attention of sampled rows")
    check_compress(hl, dev, p, [0])
    check_csa_rows(hl, dev, p, [(0, 0), (7, 0), (15, 0)], unfused=False)


def test_csa_decode_128k_unfused(csa):
    hosts, dev, st = run_workload("csa_decode_128k", indexer="unfused")
    (p, hl), = hosts
    assert "indexer_scores" in st.order and "topk" in st.order
    say("csa_decode_128k, separate calls: scores, top-k and attention of sampled rows")
    check_csa_rows(hl, dev, p, [(0, 0), (9, 0)], unfused=True)


def test_hca_decode_1m(csa):
    hosts, dev, st = run_workload("hca_decode_1m")
    (p, hl), = hosts
    say("hca_decode_1m: pooled fp8 entry and attention of every row")
    check_compress(hl, dev, p, [0])
    check_hca_rows(hl, dev, p, [(b, 0) for b in range(hl["wl"].B)])


def test_csa_prefill_256k(csa):
    hosts, dev, st = run_workload("csa_prefill_256k")
    (p, hl), = hosts
    assert "indexer_topk" in st.order
    say("csa_prefill_256k: pooled chunk entries, fused top-k and attention of sampled rows")
    check_compress(hl, dev, p, [0, 511, 1023])
    check_csa_rows(hl, dev, p, [(0, 0), (0, 2047), (0, 4095)], unfused=False)


def test_layer_pair_1m_split(csa):
    hosts, dev, st = run_workload("pair_1m_split")
    layers = dict(hosts)
    say("pair_1m_split: every layer's pooled entries and sampled rows")
    check_compress(layers["csa_decode."], dev, "csa_decode.", [0])
    check_csa_rows(layers["csa_decode."], dev, "csa_decode.", [(3, 0)], unfused=False)
    check_compress(layers["csa_chunk."], dev, "csa_chunk.", [0, 511])
    check_csa_rows(layers["csa_chunk."], dev, "csa_chunk.", [(0, 0), (0, 2047)], unfused=False)
    check_compress(layers["hca_decode."], dev, "hca_decode.", [0])
    check_hca_rows(layers["hca_decode."], dev, "hca_decode.", [(0, 0), (3, 0)])
    check_compress(layers["hca_chunk."], dev, "hca_chunk.", [0, 15])
    check_hca_rows(layers["hca_chunk."], dev, "hca_chunk.", [(0, 0), (0, 1000), (0, 2047)])


def run_pair_packed():
    """The 1M layer pair's mixed step as bench.py times it: 4 decode rows and the
    2048-token chunk packed into one varlen call per op.  Returns the per-layer host
    inputs and, per layer part, views of the packed device state in the per-part
    layout the checks read ([B, ...] per part)."""
    wls = workloads()
    hosts = [(prefix, bench.host_layer(wls[w])) for prefix, w in bench.LAYERS["pair_1m_split"]]
    hd = {prefix.rstrip("."): hl for prefix, hl in hosts}
    st = bench.Step("pair_1m", 0)
    dev = {}
    for kind in ("csa", "hca"):
        dec, ch = hd[kind + "_decode"], hd[kind + "_chunk"]
        pk = bench.pack_layer(dec, ch)
        bench.add_varlen_layer(st, dec, ch, kind + ".")
        dev.update(bench.device_packed(pk, kind + ".", kind, dec["wl"].k))
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in dev.items()}
    say(f"pair_1m (packed): calls {st.order}")
    st.run(dev)
    torch.cuda.synchronize()
    views = {}
    for kind in ("csa", "hca"):
        p = kind + "."
        nd, T = hd[kind + "_decode"]["wl"].B, hd[kind + "_chunk"]["wl"].T_q
        for part, sb, rows, shape_bt in (("_decode.", slice(0, nd), slice(0, nd), (nd, 1)),
                                         ("_chunk.", slice(nd, nd + 1), slice(nd, nd + T), (1, T))):
            v = {kind + part + n: dev[p + n][sb] for n in ("ck", "cv") if dev[p + n] is not None}
            for n in ("cks", "cvs"):
                v[kind + part + n] = None if dev[p + n] is None else dev[p + n][sb]
            out = dev[p + "out"][rows]
            v[kind + part + "out"] = out.reshape(shape_bt + tuple(out.shape[1:]))
            if kind == "csa":
                ix = dev[p + "idx"][rows]
                v[kind + part + "idx"] = ix.reshape(shape_bt + tuple(ix.shape[1:]))
            views.update(v)
    return hosts, views


def test_layer_pair_1m(csa):
    hosts, dev = run_pair_packed()
    layers = dict(hosts)
    say("pair_1m (packed varlen calls): every layer's pooled entries and sampled rows")
    check_compress(layers["csa_decode."], dev, "csa_decode.", [0])
    check_csa_rows(layers["csa_decode."], dev, "csa_decode.", [(0, 0), (3, 0)], unfused=False)
    check_compress(layers["csa_chunk."], dev, "csa_chunk.", [0, 511])
    check_csa_rows(layers["csa_chunk."], dev, "csa_chunk.", [(0, 0), (0, 1023), (0, 2047)], unfused=False)
    check_compress(layers["hca_decode."], dev, "hca_decode.", [0])
    check_hca_rows(layers["hca_decode."], dev, "hca_decode.", [(0, 0), (3, 0)])
    check_compress(layers["hca_chunk."], dev, "hca_chunk.", [0, 15])
    check_hca_rows(layers["hca_chunk."], dev, "hca_chunk.", [(0, 0), (0, 1000), (0, 2047)])
