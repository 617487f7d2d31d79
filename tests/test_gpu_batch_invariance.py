"""GPU tests of the batch-invariant attention calls (csa_sparse_attn_batch_invariant,
hca_dense_attn_batch_invariant).

These calls cut each row's key list into pieces whose length depends on the list length
alone and fold the pieces' states in order.  Calls with many rows fold inside one block per
row; calls with few rows run the pieces as blocks of their own and fold their partials in a
second kernel.  Slicing a batch so that both forms occur must give the same bits.

A row's out and lse must be bit-identical whether it is computed in a large batch, alone,
or in prefill chunks of another length; and the results must match the oracle to the same
tolerance as the plain calls.  Inputs are the seeded synthetic attention inputs of the
parity tests (normal queries and keys, random visible top-k lists, raw windows).
"""
import numpy as np
import pytest
import torch

from csa_synth import attn_inputs, random_topk_idx
from gpu_helpers import attention_tolerance, h, h_bf16, say, t_f32, t_i32, t_kv, t_u8
from oracle.attention import decode_kv, dense_attn, sparse_attn
from oracle.formats import bf16_decode
from oracle.indexer import nvis

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _dev(x, io, ckv):
    q = t_kv(x["q"], io)
    if ckv == "fp8":
        ck, cv, cks, cvs = t_u8(x["cK"]), t_u8(x["cV"]), t_f32(x["cK_scale"]), t_f32(x["cV_scale"])
    else:
        ck, cv, cks, cvs = t_kv(x["cK"], ckv), t_kv(x["cV"], ckv), None, None
    return q, ck, cv, cks, cvs, t_kv(x["Kw"], io), t_kv(x["Vw"], io)


def _oracle_inputs(x, io, ckv):
    return (decode_kv(x["q"], io), decode_kv(x["cK"], ckv, x["cK_scale"]),
            decode_kv(x["cV"], ckv, x["cV_scale"]), decode_kv(x["Kw"], io), decode_kv(x["Vw"], io))


def _host(out, io):
    return bf16_decode(h_bf16(out)) if io == "bf16" else h(out).astype(np.float64)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _check_oracle(out, lse_g, O, lse, io):
    diff = np.abs(_host(out, io) - O)
    say(f"  max-abs err vs oracle {diff.max():.3e}")
    assert np.all(diff <= attention_tolerance(O, io))
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(h(lse_g)), fin)
    if fin.any():
        assert np.abs(h(lse_g)[fin] - lse[fin]).max() <= (1e-3 if io == "bf16" else 1e-5)


SPARSE_DECODE = [
    # io, ckv, B, H, cap, k, W, pos0 (m = 4); one query per sequence
    ("bf16", "bf16", 6, 64, 1200, 1024, 128, [4799, 4000, 2000, 4100, 1500, 4799]),
    ("bf16", "fp8", 5, 128, 800, 512, 128, [3199, 1000, 3000, 2500, 700]),
    ("f32", "f32", 4, 32, 700, 600, 64, [2799, 2700, 1800, 2400]),
]


@pytest.mark.parametrize("io,ckv,B,H,cap,k,W,pos", SPARSE_DECODE)
def test_sparse_decode_rows_ignore_the_batch(csa, io, ckv, B, H, cap, k, W, pos):
    say(f"batch-invariant sparse decode io={io} ckv={ckv} B={B} H={H} k={k}")
    pos = np.array(pos, np.int32)
    raw0 = (pos + 1 - W).astype(np.int32)
    x = attn_inputs(B, 1, H, cap, W, io, ckv, seed=k + B)
    idx = random_topk_idx(np.minimum(nvis(pos[:, None], 4), cap), k, cap, seed=B)
    q, ck, cv, cks, cvs, kw, vw = _dev(x, io, ckv)
    lse_all = torch.empty((B, 1, H), device="cuda")
    out_all = csa.csa_sparse_attn_batch_invariant(q, ck, cv, t_i32(idx), kw, vw, t_i32(raw0), t_i32(pos), W,
                                                  ck_scale=cks, cv_scale=cvs, lse=lse_all)
    torch.cuda.synchronize()
    oq, oK, oV, oKw, oVw = _oracle_inputs(x, io, ckv)
    _check_oracle(out_all, lse_all, *sparse_attn(oq, oK, oV, idx, oKw, oVw, raw0, pos, W), io)
    for b in range(B):
        sl = slice(b, b + 1)
        lse_1 = torch.empty((1, 1, H), device="cuda")
        out_1 = csa.csa_sparse_attn_batch_invariant(
            q[sl], ck[sl], cv[sl], t_i32(idx[sl]), kw[sl], vw[sl], t_i32(raw0[sl]), t_i32(pos[sl]), W,
            ck_scale=None if cks is None else cks[sl], cv_scale=None if cvs is None else cvs[sl], lse=lse_1)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_1), _bits(out_all[sl])), b
        assert np.array_equal(_bits(lse_1), _bits(lse_all[sl])), b


def _chunks_equal_whole(call, T, cuts, q, qpos, lse_whole, out_whole, H):
    """Run the same queries as consecutive chunks (cut at `cuts`) and compare bits."""
    edges = [0] + list(cuts) + [T]
    for a, e in zip(edges[:-1], edges[1:]):
        lse_c = torch.empty((q.shape[0], e - a, H), device="cuda")
        out_c = call(q[:, a:e].contiguous(), t_i32(qpos + a), lse_c)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_c), _bits(out_whole[:, a:e])), (a, e)
        assert np.array_equal(_bits(lse_c), _bits(lse_whole[:, a:e])), (a, e)


@pytest.mark.parametrize("io,ckv,T,H,mp,cap,W,pos,cuts", [
    ("bf16", "bf16", 512, 64, 16, 300, 64, 4200, [256]),      # the plain call takes another kernel here
    ("bf16", "fp8", 300, 32, 8, 700, 16, 4000, [1, 77, 200]),
    ("f32", "f32", 130, 16, 32, 200, 40, 5000, [64]),
    # many pieces: the whole chunk folds them inside one block per row, the short chunks
    # run them as blocks of their own and fold their partials in a second kernel
    ("bf16", "fp8", 200, 64, 4, 700, 128, 2300, [20, 40, 60, 80, 100, 150, 180]),
    ("f32", "fp8", 160, 32, 4, 700, 64, 2500, [10, 130]),
])
def test_dense_prefill_rows_ignore_the_chunking(csa, io, ckv, T, H, mp, cap, W, pos, cuts):
    say(f"batch-invariant dense prefill io={io} ckv={ckv} T={T} H={H} m'={mp} cuts={cuts}")
    L_raw = T + W
    pos0 = np.array([pos], np.int32)
    raw0 = (pos0 + T - L_raw).astype(np.int32)
    x = attn_inputs(1, T, H, cap, L_raw, io, ckv, seed=T + cap)
    q, ck, cv, cks, cvs, kw, vw = _dev(x, io, ckv)

    def call(qq, qp, lse):
        return csa.hca_dense_attn_batch_invariant(qq, ck, cv, mp, kw, vw, t_i32(raw0), qp, W,
                                                  ck_scale=cks, cv_scale=cvs, lse=lse)
    lse_all = torch.empty((1, T, H), device="cuda")
    out_all = call(q, t_i32(pos0), lse_all)
    torch.cuda.synchronize()
    oq, oK, oV, oKw, oVw = _oracle_inputs(x, io, ckv)
    _check_oracle(out_all, lse_all, *dense_attn(oq, oK, oV, mp, oKw, oVw, raw0, pos0, W), io)
    _chunks_equal_whole(call, T, cuts, q, pos0, lse_all, out_all, H)


def test_sparse_prefill_rows_ignore_the_chunking(csa):
    io, ckv, T, H, cap, k, W = "bf16", "bf16", 300, 64, 600, 100, 32
    say(f"batch-invariant sparse prefill T={T} H={H} k={k}")
    L_raw = T + W
    pos0 = np.array([2000], np.int32)
    raw0 = (pos0 + T - L_raw).astype(np.int32)
    x = attn_inputs(1, T, H, cap, L_raw, io, ckv, seed=7)
    idx = random_topk_idx(np.minimum(nvis(pos0[:, None] + np.arange(T)[None], 4), cap), k, cap, seed=3)
    q, ck, cv, cks, cvs, kw, vw = _dev(x, io, ckv)

    def call(qq, qp, lse):
        a = int(h(qp)[0] - pos0[0])
        ii = t_i32(np.ascontiguousarray(idx[:, a:a + qq.shape[1]]))
        return csa.csa_sparse_attn_batch_invariant(qq, ck, cv, ii, kw, vw, t_i32(raw0), qp, W, lse=lse)
    lse_all = torch.empty((1, T, H), device="cuda")
    out_all = call(q, t_i32(pos0), lse_all)
    torch.cuda.synchronize()
    oq, oK, oV, oKw, oVw = _oracle_inputs(x, io, ckv)
    _check_oracle(out_all, lse_all, *sparse_attn(oq, oK, oV, idx, oKw, oVw, raw0, pos0, W), io)
    _chunks_equal_whole(call, T, [100, 101], q, pos0, lse_all, out_all, H)


def test_long_list_and_plain_call_agree(csa):
    """A 128K-context decode list (2048 selected + 128 window keys) over 16 sequences: the
    batch-invariant call agrees with the plain call to the attention tolerance, and each of
    three sampled rows alone gives the batch's bits."""
    B, H, cap, k, W = 16, 64, 32768, 2048, 128
    say(f"batch-invariant vs plain, B={B} k={k} cap={cap}")
    pos = np.full(B, 131071, np.int32)
    raw0 = (pos + 1 - W).astype(np.int32)
    x = attn_inputs(B, 1, H, cap, W, "bf16", "fp8", seed=11)
    idx = random_topk_idx(np.minimum(nvis(pos[:, None], 4), cap), k, cap, seed=5)
    q, ck, cv, cks, cvs, kw, vw = _dev(x, "bf16", "fp8")
    args = (q, ck, cv, t_i32(idx), kw, vw, t_i32(raw0), t_i32(pos), W)
    out_bi = csa.csa_sparse_attn_batch_invariant(*args, ck_scale=cks, cv_scale=cvs)
    out_pl = csa.csa_sparse_attn(*args, ck_scale=cks, cv_scale=cvs)
    torch.cuda.synchronize()
    a, b = bf16_decode(h_bf16(out_bi)), bf16_decode(h_bf16(out_pl))
    assert np.all(np.abs(a - b) <= 2e-2 * np.maximum(np.abs(b), 1.0))
    for r in (0, 7, 15):
        sl = slice(r, r + 1)
        o1 = csa.csa_sparse_attn_batch_invariant(q[sl], ck[sl], cv[sl], t_i32(idx[sl]), kw[sl], vw[sl],
                                                 t_i32(raw0[sl]), t_i32(pos[sl]), W, ck_scale=cks[sl],
                                                 cv_scale=cvs[sl])
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o1), _bits(out_bi[sl])), r


@pytest.mark.parametrize("dense", [False, True])
def test_varlen_mixed_decode_and_prefill(csa, dense):
    """Four decode rows (sequences 0-3) and a 200-query prefill chunk (sequence 4) in one
    varlen call: each part's rows equal, bit for bit, the batch-invariant call on its own
    sequences, and the oracle within the attention tolerance."""
    io, ckv, H, cap, W, T, k, m, mp = "bf16", "fp8", 64, 800, 64, 200, 256, 4, 16
    say(f"varlen mixed step dense={dense}: 4 decode rows + {T}-query chunk")
    dec_pos = np.array([3199, 2000, 1500, 3100], np.int32)
    c_pos0 = 2500
    L_raw = T + W
    pos0 = np.concatenate([dec_pos, [c_pos0]]).astype(np.int32)
    last = np.concatenate([dec_pos, [c_pos0 + T - 1]])
    raw0 = (last + 1 - L_raw).astype(np.int32)
    x = attn_inputs(5, T, H, cap, L_raw, io, ckv, seed=123)
    q, ck, cv, cks, cvs, kw, vw = _dev(x, io, ckv)
    cu_rows = np.array([0, 1, 2, 3, 4, 4 + T], np.int32)
    qv = torch.cat([q[0:4, 0], q[4, :T]]).contiguous()
    lse_v = torch.empty((4 + T, H), device="cuda")
    oq, oK, oV, oKw, oVw = _oracle_inputs(x, io, ckv)
    if dense:
        out_v = csa.hca_dense_attn_varlen(qv, ck, cv, mp, kw, vw, t_i32(raw0), t_i32(cu_rows), t_i32(pos0), W,
                                          ck_scale=cks, cv_scale=cvs, lse=lse_v)
    else:
        idx_dec = random_topk_idx(np.minimum(nvis(dec_pos[:, None], m), cap), k, cap, seed=1)      # [4, 1, k]
        idx_c = random_topk_idx(np.minimum(nvis(c_pos0 + np.arange(T)[None], m), cap), k, cap, seed=2)  # [1, T, k]
        idx_v = np.ascontiguousarray(np.concatenate([idx_dec[:, 0], idx_c[0]]))
        out_v = csa.csa_sparse_attn_varlen(qv, ck, cv, t_i32(idx_v), kw, vw, t_i32(raw0), t_i32(cu_rows),
                                           t_i32(pos0), W, ck_scale=cks, cv_scale=cvs, lse=lse_v)
    parts = [(slice(0, 4), slice(0, 1), slice(0, 4)), (slice(4, 5), slice(0, T), slice(4, 4 + T))]
    for pi, (sb, st_, sr) in enumerate(parts):
        lse_p = torch.empty((sb.stop - sb.start, st_.stop, H), device="cuda")
        qq = q[sb, st_].contiguous()
        kwargs = dict(ck_scale=cks[sb], cv_scale=cvs[sb], lse=lse_p)
        if dense:
            out_p = csa.hca_dense_attn_batch_invariant(qq, ck[sb], cv[sb], mp, kw[sb], vw[sb], t_i32(raw0[sb]),
                                                       t_i32(pos0[sb]), W, **kwargs)
            O, lse = dense_attn(oq[sb, st_], oK[sb], oV[sb], mp, oKw[sb], oVw[sb], raw0[sb], pos0[sb], W)
        else:
            ip = idx_dec if pi == 0 else idx_c
            out_p = csa.csa_sparse_attn_batch_invariant(qq, ck[sb], cv[sb], t_i32(ip), kw[sb], vw[sb],
                                                        t_i32(raw0[sb]), t_i32(pos0[sb]), W, **kwargs)
            O, lse = sparse_attn(oq[sb, st_], oK[sb], oV[sb], ip, oKw[sb], oVw[sb], raw0[sb], pos0[sb], W)
        torch.cuda.synchronize()
        got = out_v[sr].reshape(out_p.shape)
        assert np.array_equal(_bits(got), _bits(out_p)), pi
        assert np.array_equal(_bits(lse_v[sr].reshape(lse_p.shape)), _bits(lse_p)), pi
        _check_oracle(got, lse_v[sr].reshape(lse_p.shape), O, lse, io)
