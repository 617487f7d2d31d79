"""A mixed decode + prefill step of a CSA / HCA layer pair through the varlen calls.

Four sequences decode one token each (some of them completing a block) and a fifth runs a
prefill chunk, all in one call per operation: csa_compress_kv_varlen pools every block the
step completes, csa_indexer_topk_varlen selects the entries of every query row, and
csa_sparse_attn_varlen / hca_dense_attn_varlen attend.  Checks:
  * each varlen call equals, bit for bit, the plain calls on the sequences one at a time
    (csa_compress_kv per sequence, csa_indexer_topk per part, the batch-invariant attention
    per part);
  * the chain against the oracle: stored entries within the compression tolerance (fp8
    E4M3 per-entry scales), indices identical to the oracle's top-k on exact indexer scores
    (dyadic MXFP4 operands), attention outputs within the attention tolerance of the
    oracle's chain, which pools the same raw rows in fp64 and stores them by its own rule.
"""
import numpy as np
import pytest
import torch

from csa_synth import compress_inputs, indexer_inputs, normal_f32, normal_kv, streams
from gpu_helpers import (attention_tolerance, compress_tolerance, h, h_bf16, say, t_bf16, t_f32, t_i32,
                         t_u8)
from oracle.attention import decode_kv, dense_attn, sparse_attn
from oracle.compress import compress_values, store
from oracle.formats import bf16_decode, e4m3_decode
from oracle.indexer import indexer_scores, nvis
from oracle.topk import topk

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


class Step:
    """Positions of the step: sequences 0-3 decode at dec_pos, sequence 4 runs a chunk of T
    queries from c_pos0; every sequence's newest token sits in the last row of its raw
    window buffer of L_raw rows."""

    def __init__(self, dec_pos, c_pos0, T, W):
        self.dec_pos = np.asarray(dec_pos, np.int32)
        self.c_pos0, self.T, self.W = c_pos0, T, W
        self.B = len(dec_pos) + 1
        self.L_raw = T + W
        self.pos0 = np.concatenate([self.dec_pos, [c_pos0]]).astype(np.int32)
        self.last = np.concatenate([self.dec_pos, [c_pos0 + T - 1]]).astype(np.int64)
        self.raw0 = (self.last + 1 - self.L_raw).astype(np.int32)
        self.n_rows = len(dec_pos) + T
        self.cu_rows = np.array(list(range(len(dec_pos) + 1)) + [self.n_rows], np.int32)

    def new_blocks(self, m):
        """Per sequence: (first raw row, first entry, count) of the blocks the step completes."""
        out = []
        for b in range(self.B):
            first_tok = self.last[b] if b < self.B - 1 else self.c_pos0
            e_lo = (first_tok + m) // m - 1            # first block ending at or after first_tok
            e_hi = (self.last[b] + 1) // m              # blocks ending at or before last
            n = max(0, e_hi - e_lo)
            out.append((int(e_lo * m - self.raw0[b]), int(e_lo), int(n)))
        return out


def _cache(B, cap, seed, ro):
    """An fp8 cache of N(0,1) entries (1% x8 outliers) stored by the oracle's rule."""
    rk, rv = streams(141, seed, 2)
    cK, cKs = store(normal_f32(rk, (B, cap, D), ro).astype(np.float64), "fp8")
    cV, cVs = store(normal_f32(rv, (B, cap, D), ro).astype(np.float64), "fp8")
    return cK, cKs, cV, cVs


def _compress_both(csa, s, m, kv, cache):
    """GPU: csa_compress_kv_varlen into a copy of the cache, and csa_compress_kv per sequence
    into another; oracle: the fp64 pool of the same rows stored by its rule into a third."""
    cK, cKs, cV, cVs = cache
    blocks = s.new_blocks(m)
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in blocks])]).astype(np.int32)
    row0 = np.array([r for r, _, _ in blocks], np.int32)
    entry0 = np.array([e for _, e, _ in blocks], np.int32)
    assert np.all(row0 >= 0) and np.all(row0 + np.diff(cu) * m <= s.L_raw)
    dev = [t_u8(cK), t_u8(cV), t_f32(cKs), t_f32(cVs)]
    ref = [x.clone() for x in dev]
    Kw, Vw = t_bf16(kv["K"]), t_bf16(kv["V"])
    lg = t_f32(kv["logits"])
    csa.csa_compress_kv_varlen(Kw, Vw, lg, m, dev[0], dev[1], t_i32(cu), t_i32(row0), t_i32(entry0), int(cu[-1]),
                               k_scale_out=dev[2], v_scale_out=dev[3])
    for b, (r, e, n) in enumerate(blocks):
        if n:
            csa.csa_compress_kv(Kw[b:b + 1], Vw[b:b + 1], lg[b:b + 1], m, ref[0][b:b + 1], ref[1][b:b + 1],
                                ref[2][b:b + 1], ref[3][b:b + 1], L=n * m, row0=r, entry0=e)
    torch.cuda.synchronize()
    for a, b_ in zip(dev, ref):
        assert torch.equal(a, b_)
    # the oracle's cache after the same pooling
    oK, oKs, oV, oVs = cK.copy(), cKs.copy(), cV.copy(), cVs.copy()
    Kf, Vf = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    for b, (r, e, n) in enumerate(blocks):
        if not n:
            continue
        sl = slice(r, r + n * m)
        Kh, Vh = compress_values(Kf[b:b + 1, sl], Vf[b:b + 1, sl], kv["logits"][b:b + 1, sl], m)
        (ck_, cks_), (cv_, cvs_) = store(Kh, "fp8"), store(Vh, "fp8")
        oK[b, e:e + n], oKs[b, e:e + n], oV[b, e:e + n], oVs[b, e:e + n] = ck_[0], cks_[0], cv_[0], cvs_[0]
        # stored GPU entries against the oracle's, within the compression tolerance
        amax = np.abs(np.stack([Kf[b, sl], Vf[b, sl]])).reshape(2, n, m, D).max(axis=(2, 3))
        for w, X, codes, sc in ((0, Kh[0], dev[0], dev[2]), (1, Vh[0], dev[1], dev[3])):
            eps = (m + 4) * 2.0 ** -24 * amax[w][:, None]
            gs = h(sc[b, e:e + n]).astype(np.float64)
            g = e4m3_decode(h(codes[b, e:e + n])) * gs[:, None]
            oc, osc = store(X, "fp8")
            o = e4m3_decode(oc) * osc[:, None].astype(np.float64)
            assert np.all(np.abs(g - o) <= compress_tolerance(X, "fp8", eps, osc)), (b, w)
    say(f"  compression m={m}: {int(cu[-1])} entries, varlen == per-sequence calls, within tolerance of the oracle")
    return dev, (oK, oKs, oV, oVs)


@pytest.mark.parametrize("dec_pos,c_pos0,T", [
    ([3199, 2000, 1503, 3071], 2560, 150),      # blocks completed by some decode rows, chunk aligned
    ([3263, 3327, 3391, 3455], 2501, 77),       # every decode row completes both blocks; ragged chunk
    ([3199, 2999, 3071, 2047], 2816, 300),      # 304 rows: the plain dense call's many-query path
])
def test_mixed_step(csa, dec_pos, c_pos0, T):
    H, W, m, mp, k, H_I, d_I = 64, 64, 4, 64, 256, 8, 128
    s = Step(dec_pos, c_pos0, T, W)
    cap = int(nvis(s.last.max(), m))
    cap_h = int(nvis(s.last.max(), mp))
    say(f"mixed varlen step: {len(dec_pos)} decode rows + {T}-query chunk, cap {cap} / {cap_h}")
    (ro,) = streams(142, c_pos0, 1)
    kv_c = compress_inputs(s.B, s.L_raw, "bf16", seed=c_pos0, tag=143, outliers=True)
    kv_h = compress_inputs(s.B, s.L_raw, "bf16", seed=c_pos0, tag=144, outliers=True)
    rq, rqh = streams(145, c_pos0, 2)
    q_c = normal_kv(rq, (s.n_rows, H, D), "bf16")
    q_h = normal_kv(rqh, (s.n_rows, H, D), "bf16")
    ix = indexer_inputs(1, s.n_rows, cap, H_I, d_I, seed=c_pos0)
    ixk = indexer_inputs(s.B, 1, cap, H_I, d_I, seed=c_pos0 + 1)
    qc, qe, w = ix["q_codes"][0], ix["q_e8m0"][0], ix["w"][0]
    kc, ke = ixk["k_codes"], ixk["k_e8m0"]

    # --- CSA layer: compression, selection, sparse attention
    dc, oc = _compress_both(csa, s, m, kv_c, _cache(s.B, cap, 1, ro))
    d_ix = (t_u8(qc), t_u8(qe), t_f32(w), t_u8(kc), t_u8(ke))
    idx = csa.csa_indexer_topk_varlen(*d_ix, t_i32(s.cu_rows), t_i32(s.pos0), m, k)
    torch.cuda.synchronize()
    idx_h = h(idx)
    want = np.full((s.n_rows, k), -1, np.int32)
    for b in range(s.B):
        r = slice(s.cu_rows[b], s.cu_rows[b + 1])
        sc = indexer_scores(qc[None, r], qe[None, r], w[None, r], kc[b:b + 1], ke[b:b + 1], s.pos0[b:b + 1], m)
        want[r] = topk(sc.astype(np.float32), s.pos0[b:b + 1], m, k)[0]
        one = csa.csa_indexer_topk(t_u8(qc[None, r]), t_u8(qe[None, r]), t_f32(w[None, r]), t_u8(kc[b:b + 1]),
                                   t_u8(ke[b:b + 1]), t_i32(s.pos0[b:b + 1]), m, k)
        torch.cuda.synchronize()
        assert np.array_equal(h(one)[0], idx_h[r]), b
    assert np.array_equal(idx_h, want)
    say("  selection: varlen == per-sequence csa_indexer_topk == oracle top-k")
    for inv in (True, False):
        _attend(csa, s, False, inv, q_c, dc, oc, kv_c, idx, want, m, W, H)

    # --- HCA layer: compression (long blocks), dense attention
    dh, oh = _compress_both(csa, s, mp, kv_h, _cache(s.B, cap_h, 2, ro))
    for inv in (True, False):
        _attend(csa, s, True, inv, q_h, dh, oh, kv_h, None, None, mp, W, H)


def _attend(csa, s, dense, inv, q, dcache, ocache, kv, idx, idx_o, m, W, H):
    """Both layers' varlen attention over the step's rows; invariant mode: bit-equal to the
    batch-invariant call on each part; both modes: within tolerance of the oracle."""
    ck, cv, cks, cvs = dcache
    kw, vw = t_bf16(kv["K"]), t_bf16(kv["V"])
    qv = t_bf16(q)
    lse_v = torch.empty((s.n_rows, H), device="cuda")
    cu, p0 = t_i32(s.cu_rows), t_i32(s.pos0)
    if dense:
        out = csa.hca_dense_attn_varlen(qv, ck, cv, m, kw, vw, t_i32(s.raw0), cu, p0, W, ck_scale=cks, cv_scale=cvs,
                                        invariant=inv, lse=lse_v)
    else:
        out = csa.csa_sparse_attn_varlen(qv, ck, cv, idx, kw, vw, t_i32(s.raw0), cu, p0, W, ck_scale=cks,
                                         cv_scale=cvs, invariant=inv, lse=lse_v)
    torch.cuda.synchronize()
    oK, oKs, oV, oVs = ocache
    cK_o, cV_o = decode_kv(oK, "fp8", oKs), decode_kv(oV, "fp8", oVs)
    Kw_o, Vw_o = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    qo = bf16_decode(q)
    nd = s.B - 1
    # decode part (sequences 0..nd-1, one row each) and chunk part (sequence nd)
    for sb, rows, T in ((slice(0, nd), slice(0, nd), 1), (slice(nd, s.B), slice(nd, s.n_rows), s.T)):
        nb = sb.stop - sb.start
        qo_p = qo[rows].reshape(nb, T, H, D)
        got = out[rows].reshape(nb, T, H, D)
        lse_g = lse_v[rows].reshape(nb, T, H)
        if dense:
            O, lse = dense_attn(qo_p, cK_o[sb], cV_o[sb], m, Kw_o[sb], Vw_o[sb], s.raw0[sb], s.pos0[sb], W)
        else:
            O, lse = sparse_attn(qo_p, cK_o[sb], cV_o[sb], idx_o[rows].reshape(nb, T, -1), Kw_o[sb], Vw_o[sb],
                                 s.raw0[sb], s.pos0[sb], W)
        if inv:
            qq = qv[rows].reshape(nb, T, H, D)
            lse_p = torch.empty((nb, T, H), device="cuda")
            kw_ = dict(ck_scale=cks[sb], cv_scale=cvs[sb], lse=lse_p)
            if dense:
                ref = csa.hca_dense_attn_batch_invariant(qq, ck[sb], cv[sb], m, kw[sb], vw[sb], t_i32(s.raw0[sb]),
                                                         t_i32(s.pos0[sb]), W, **kw_)
            else:
                ip = idx[rows].reshape(nb, T, -1).contiguous()
                ref = csa.csa_sparse_attn_batch_invariant(qq, ck[sb], cv[sb], ip, kw[sb], vw[sb],
                                                          t_i32(s.raw0[sb]), t_i32(s.pos0[sb]), W, **kw_)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(got), _bits(ref))
            assert np.array_equal(_bits(lse_g), _bits(lse_p))
        diff = np.abs(bf16_decode(h_bf16(got)) - O)
        say(f"  {'dense' if dense else 'sparse'} attention ({'invariant' if inv else 'plain'}), "
            f"{'decode' if T == 1 else 'chunk'} rows{': == batch-invariant call' if inv else ''}; "
            f"max-abs err vs oracle {diff.max():.3e}")
        assert np.all(diff <= attention_tolerance(O, "bf16"))
        fin = np.isfinite(lse)
        g = h(lse_g)
        assert np.array_equal(np.isfinite(g), fin)
        assert np.abs(g[fin] - lse[fin]).max() <= 1e-3


@pytest.mark.parametrize("H,mp,lens", [
    (64, 16, [1, 3, 0, 4, 5, 300]),       # pieces for 1, 3, 4 rows; tiles for 5 and 300; an empty sequence
    (32, 32, [8, 2, 260, 9, 1]),          # H = 32: 8 queries per tile
    (128, 16, [2, 1, 270, 3]),            # H = 128: 2 queries per tile
])
def test_dense_varlen_many_query_mix(csa, H, mp, lens):
    """The plain dense varlen call over >= 256 rows (the many-query kernel with key pieces for
    short sequences and their merge) against the oracle, row by row, with fp8 entries."""
    W = 64
    B = len(lens)
    lens = np.array(lens)
    rng = streams(146, H, 1)[0]
    pos0 = rng.integers(1200, 2400, size=B).astype(np.int32)
    last = pos0 + np.maximum(lens, 1) - 1
    L_raw = int(lens.max()) + W
    raw0 = (last + 1 - L_raw).astype(np.int32)
    cap = int(nvis(last.max(), mp))
    say(f"dense varlen many-query H={H} m'={mp} rows per sequence {list(lens)}")
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n_rows = int(cu[-1])
    assert n_rows >= 256
    (ro,) = streams(147, H, 1)
    cK, cKs, cV, cVs = _cache(B, cap, 3, ro)
    kv = compress_inputs(B, L_raw, "bf16", seed=H, tag=148, outliers=True)
    q = normal_kv(streams(149, H, 1)[0], (n_rows, H, D), "bf16")
    lse_v = torch.empty((n_rows, H), device="cuda")
    out = csa.hca_dense_attn_varlen(t_bf16(q), t_u8(cK), t_u8(cV), mp, t_bf16(kv["K"]), t_bf16(kv["V"]),
                                    t_i32(raw0), t_i32(cu), t_i32(pos0), W, ck_scale=t_f32(cKs),
                                    cv_scale=t_f32(cVs), invariant=False, lse=lse_v)
    torch.cuda.synchronize()
    got, lse_g = bf16_decode(h_bf16(out)), h(lse_v)
    cK_o, cV_o = decode_kv(cK, "fp8", cKs), decode_kv(cV, "fp8", cVs)
    Kw_o, Vw_o = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    qo = bf16_decode(q)
    worst = 0.0
    for b in range(B):
        r = slice(cu[b], cu[b + 1])
        T = int(lens[b])
        if T == 0:
            continue
        O, lse = dense_attn(qo[r].reshape(1, T, H, D), cK_o[b:b + 1], cV_o[b:b + 1], mp, Kw_o[b:b + 1],
                            Vw_o[b:b + 1], raw0[b:b + 1], pos0[b:b + 1], W)
        diff = np.abs(got[r].reshape(O.shape) - O)
        worst = max(worst, diff.max())
        assert np.all(diff <= attention_tolerance(O, "bf16")), b
        g = lse_g[r].reshape(lse.shape)
        fin = np.isfinite(lse)
        assert np.array_equal(np.isfinite(g), fin), b
        assert np.abs(g[fin] - lse[fin]).max() <= 1e-3, b
    say(f"  every row within tolerance of the oracle (max-abs err {worst:.3e})")
