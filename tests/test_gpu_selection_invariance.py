"""Batch invariance of the indexer scores and of the selections built on them.

A query row's scores (and therefore its top-k) must not depend on the batch around it: the
row computed in one prefill chunk, in chunks cut at odd offsets (the row then sits in another
slot of the matrix-core tile), alone as a decoding row (another kernel: the per-slice pass of
the decode path), or in a batch of several sequences must give the same bits.  The inputs
make the scores inexact in fp32 (real-valued head weights, block scales spread over 2^-17 ..
2^13), so any difference in the summation order would show.
"""
import numpy as np
import pytest
import torch

from csa_synth import compress_inputs, indexer_inputs, streams
from gpu_helpers import h, say, t_bf16, t_f32, t_i32, t_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _inexact(B, T, cap, H_I, d_I, seed):
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=seed)
    (r,) = streams(131, seed, 1)
    x["w"] = r.uniform(0.05, 3.0, size=x["w"].shape).astype(np.float32)
    x["q_e8m0"] = r.integers(110, 140, size=x["q_e8m0"].shape).astype(np.uint8)
    x["k_e8m0"] = r.integers(110, 140, size=x["k_e8m0"].shape).astype(np.uint8)
    return x


def _rows(x, sl_b, sl_t):
    return {k: np.ascontiguousarray(v[sl_b, sl_t]) if k in ("q_codes", "q_e8m0", "w") else v[sl_b]
            for k, v in x.items()}


def _dev(x):
    return (t_u8(x["q_codes"]), t_u8(x["q_e8m0"]), t_f32(x["w"]), t_u8(x["k_codes"]), t_u8(x["k_e8m0"]))


@pytest.mark.parametrize("H_I,d_I,cap,T,P,k", [
    (8, 128, 12000, 40, 47000, 500),     # decoding rows take the per-slice path (cap >= 8192)
    (4, 64, 3000, 37, 11000, 100),       # 4 queries per tile
    (16, 256, 9000, 11, 35000, 300),     # one query per tile, two contraction steps
])
def test_rows_ignore_the_batch(csa, H_I, d_I, cap, T, P, k):
    m = 4
    say(f"indexer / selection batch invariance H_I={H_I} d_I={d_I} cap={cap} T={T}")
    x = _inexact(1, T, cap, H_I, d_I, seed=cap + T)
    pos = np.array([P], np.int32)
    whole = h(csa.csa_indexer_scores(*_dev(x), t_i32(pos), m))
    sel_whole = h(csa.csa_indexer_topk(*_dev(x), t_i32(pos), m, k))
    torch.cuda.synchronize()
    nv = np.minimum((P + np.arange(T) + 1) // m, cap)
    with np.errstate(over="ignore"):   # scores beyond fp16's range become inf: still unequal
        assert not np.array_equal(whole[0, 0, :nv[0]].astype(np.float64),
                                  whole[0, 0, :nv[0]].astype(np.float16).astype(np.float64))   # a real spread

    def same_scores(got, rows):
        for gi, i in enumerate(rows):
            v = nv[i]
            assert np.array_equal(got[gi, :v].view(np.uint32), whole[0, i, :v].view(np.uint32)), i

    # prefill chunks cut at odd offsets: the rows move to other tile slots
    for a, e in [(0, 3), (3, 20), (20, T), (1, 2), (5, 6)]:
        if a >= T:
            continue
        e = min(e, T)
        xs = _rows(x, slice(0, 1), slice(a, e))
        pa = np.array([P + a], np.int32)
        g = h(csa.csa_indexer_scores(*_dev(xs), t_i32(pa), m))
        sel = h(csa.csa_indexer_topk(*_dev(xs), t_i32(pa), m, k))
        torch.cuda.synchronize()
        same_scores(g[0], range(a, e))
        assert np.array_equal(sel[0], sel_whole[0, a:e]), (a, e)

    # every row as a decoding row of its own sequence, all in one batch of T sequences
    xd = {kk: (np.ascontiguousarray(np.swapaxes(v, 0, 1)) if kk in ("q_codes", "q_e8m0", "w")
               else np.ascontiguousarray(np.broadcast_to(v, (T,) + v.shape[1:])))
          for kk, v in x.items()}
    pd = (P + np.arange(T)).astype(np.int32)
    gd = h(csa.csa_indexer_scores(*_dev(xd), t_i32(pd), m))
    seld = h(csa.csa_indexer_topk(*_dev(xd), t_i32(pd), m, k))
    kv = compress_inputs(T, 2 * m, "bf16", seed=9)
    ko = torch.zeros((T, 2, 128), dtype=torch.bfloat16, device="cuda")
    selc = h(csa.csa_compress_indexer_topk(t_bf16(kv["K"]), t_bf16(kv["V"]), t_f32(kv["logits"]), ko,
                                           torch.zeros_like(ko), None, None, *_dev(xd), t_i32(pd), m, k))
    torch.cuda.synchronize()
    same_scores(gd[:, 0], range(T))
    assert np.array_equal(seld[:, 0], sel_whole[0]) and np.array_equal(selc[:, 0], sel_whole[0])

    # a few of those decoding rows alone, and in a batch of another size
    for rows in ([0], [T - 1], [2, 5, 7]):
        xr = {kk: np.ascontiguousarray(v[rows]) for kk, v in xd.items()}
        g = h(csa.csa_indexer_scores(*_dev(xr), t_i32(pd[rows]), m))
        sel = h(csa.csa_indexer_topk(*_dev(xr), t_i32(pd[rows]), m, k))
        torch.cuda.synchronize()
        same_scores(g[:, 0], rows)
        assert np.array_equal(sel[:, 0], sel_whole[0, rows]), rows
