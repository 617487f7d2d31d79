"""GPU parity of attention over fp8 compressed caches with the real per-entry scales.

The compressor and the cache append store fp8 entries with scale = fp32(amax / 448), which is
almost never a power of two.  The kernels fold the K scale (times the logit scale) into each
logit and the V scale into P before P is rounded for the matrix core, so these cases check
that folding against the oracle, element by element, with scales the storage actually holds.

Two kinds of case:
  * stage parity: both sides read identical stored caches, quantised by the oracle's own
    per-entry E4M3 rule (oracle.compress.store) from N(0,1) entries with the 1% x8 outliers
    of the layer-pair shapes;
  * chained parity: the GPU pools the raw K/V into its fp8 cache (csa_compress_kv or a run
    of csa_kv_cache_append calls) and attends over it; the oracle pools the same raw K/V in
    fp64, stores with its rule and attends.  The stored caches may differ by one E4M3 unit
    where the pool's last bit decides a rounding (checked by the compression tests); those
    few flips move the outputs far less than the attention tolerance.
Every attention call is checked in its plain, batch-invariant and varlen form.  Tolerances:
2e-2 (bf16 I/O) / 1e-5 (fp32 I/O) plus half a unit of the output format at |O|.  (These cases
found that one bf16 rounding of P before the P*V product misses 2e-2 at |O| ~ 10 when a few
outlier values dominate a row; P now enters that product as bf16 hi + lo.)
"""
import numpy as np
import pytest
import torch

from csa_synth import compress_inputs, normal_kv, normal_f32, random_topk_idx, streams
from gpu_helpers import attention_tolerance, h, h_bf16, say, t_f32, t_i32, t_kv, t_u8
from oracle.attention import decode_kv, dense_attn, sparse_attn
from oracle.compress import compress_values, store
from oracle.formats import bf16_decode
from oracle.indexer import nvis

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _inputs(B, T, H, cap, L_raw, io, seed):
    """Queries and raw window (N(0,1) + outliers) and an fp8 cache quantised by the oracle's rule.

    fp32 I/O cases draw no outliers: the layer-pair shapes that carry them are bf16, and with
    |K| up to ~40 the fp32 logits alone are off by ~|logit| * 2^-22, which moves an output by
    more than 1e-5 whatever the kernel does."""
    rq, rck, rcv, rkw, rvw, ro = streams(71, seed, 6)
    ro = ro if io == "bf16" else None
    x = dict(q=normal_kv(rq, (B, T, H, D), io), Kw=normal_kv(rkw, (B, L_raw, D), io, ro),
             Vw=normal_kv(rvw, (B, L_raw, D), io, ro))
    x["cK"], x["cK_scale"] = store(normal_f32(rck, (B, cap, D), ro).astype(np.float64), "fp8")
    x["cV"], x["cV_scale"] = store(normal_f32(rcv, (B, cap, D), ro).astype(np.float64), "fp8")
    return x


def _host(out, io):
    return bf16_decode(h_bf16(out)) if io == "bf16" else h(out).astype(np.float64)


def _check(tag, out, lse_g, O, lse, io):
    diff = np.abs(_host(out, io) - O)
    say(f"  {tag}: max-abs err {diff.max():.3e} (|O| up to {np.abs(O).max():.1f})")
    assert np.all(diff <= attention_tolerance(O, io)), tag
    fin = np.isfinite(lse)
    g = h(lse_g)
    assert np.array_equal(np.isfinite(g), fin), tag
    if fin.any():
        assert np.abs(g[fin] - lse[fin]).max() <= (1e-3 if io == "bf16" else 1e-5), tag


def _run_all_forms(csa, dense, x, io, mid, idx, raw0, pos, W, B, T, H, O, lse):
    """The plain, batch-invariant and varlen calls on the same inputs, each against the oracle."""
    q = t_kv(x["q"], io)
    ck, cv, cks, cvs = t_u8(x["cK"]), t_u8(x["cV"]), t_f32(x["cK_scale"]), t_f32(x["cV_scale"])
    kw, vw = t_kv(x["Kw"], io), t_kv(x["Vw"], io)
    r0, p0 = t_i32(raw0), t_i32(pos)
    for form in ("plain", "batch_invariant"):
        lse_g = torch.empty((B, T, H), device="cuda")
        if dense:
            out = csa.hca_dense_attn(q, ck, cv, mid, kw, vw, r0, p0, W, ck_scale=cks, cv_scale=cvs,
                                     lse=lse_g, batch_invariant=form != "plain")
        else:
            out = csa.csa_sparse_attn(q, ck, cv, t_i32(idx), kw, vw, r0, p0, W, ck_scale=cks,
                                      cv_scale=cvs, lse=lse_g, batch_invariant=form != "plain")
        torch.cuda.synchronize()
        _check(form, out, lse_g, O, lse, io)
    # varlen: every query row of every sequence in one call, in both modes
    cu = t_i32(np.arange(B + 1, dtype=np.int32) * T)
    qv = q.reshape(B * T, H, D).contiguous()
    for inv in (True, False):
        lse_v = torch.empty((B * T, H), device="cuda")
        if dense:
            out = csa.hca_dense_attn_varlen(qv, ck, cv, mid, kw, vw, r0, cu, p0, W, ck_scale=cks, cv_scale=cvs,
                                            invariant=inv, lse=lse_v)
        else:
            iv = t_i32(idx.reshape(B * T, -1))
            out = csa.csa_sparse_attn_varlen(qv, ck, cv, iv, kw, vw, r0, cu, p0, W, ck_scale=cks, cv_scale=cvs,
                                             invariant=inv, lse=lse_v)
        torch.cuda.synchronize()
        _check(f"varlen invariant={inv}", out.reshape(B, T, H, D), lse_v.reshape(B, T, H), O, lse, io)


STAGE_DENSE = [
    # io, B, T, H, m', cap, W, pos0 of each sequence; L_raw = T + W
    ("bf16", 4, 1, 64, 128, 8192, 128, [8192 * 128 - 1] * 4),       # HCA decode at 1M
    ("bf16", 1, 512, 64, 16, 300, 64, [16 * 300 - 512]),           # HCA prefill chunk
    ("f32", 2, 1, 64, 128, 1000, 128, [1000 * 128 - 1, 700 * 128]),
    ("f32", 1, 96, 32, 32, 200, 40, [32 * 200 - 96]),
]


@pytest.mark.parametrize("io,B,T,H,mp,cap,W,pos", STAGE_DENSE)
def test_dense_over_real_scale_fp8(csa, io, B, T, H, mp, cap, W, pos):
    say(f"fp8 real scales, dense io={io} B={B} T={T} H={H} m'={mp} cap={cap} W={W}")
    pos = np.array(pos, np.int32)
    L_raw = T + W
    raw0 = (pos + T - L_raw).astype(np.int32)
    x = _inputs(B, T, H, cap, L_raw, io, seed=cap + T)
    assert np.any(np.log2(x["cK_scale"]) % 1 != 0)    # the scales are not powers of two
    q, cK, cV = decode_kv(x["q"], io), decode_kv(x["cK"], "fp8", x["cK_scale"]), decode_kv(x["cV"], "fp8", x["cV_scale"])
    O, lse = dense_attn(q, cK, cV, mp, decode_kv(x["Kw"], io), decode_kv(x["Vw"], io), raw0, pos, W)
    _run_all_forms(csa, True, x, io, mp, None, raw0, pos, W, B, T, H, O, lse)


STAGE_SPARSE = [
    # io, B, T, H, cap, k, W, pos0 (m = 4)
    ("bf16", 4, 1, 64, 8192, 1024, 128, [4 * 8192 - 1, 30000, 20000, 4 * 8192 - 1]),   # CSA decode
    ("bf16", 1, 512, 64, 1500, 128, 64, [4 * 1500 - 512]),                              # CSA chunk
    ("f32", 1, 64, 64, 900, 256, 128, [4 * 900 - 64]),
]


@pytest.mark.parametrize("io,B,T,H,cap,k,W,pos", STAGE_SPARSE)
def test_sparse_over_real_scale_fp8(csa, io, B, T, H, cap, k, W, pos):
    say(f"fp8 real scales, sparse io={io} B={B} T={T} H={H} cap={cap} k={k} W={W}")
    m = 4
    pos = np.array(pos, np.int32)
    L_raw = T + W
    raw0 = (pos + T - L_raw).astype(np.int32)
    x = _inputs(B, T, H, cap, L_raw, io, seed=cap + k)
    nv = np.minimum(nvis(pos[:, None] + np.arange(T)[None], m), cap)
    idx = random_topk_idx(nv, k, cap, seed=T + 5)
    q, cK, cV = decode_kv(x["q"], io), decode_kv(x["cK"], "fp8", x["cK_scale"]), decode_kv(x["cV"], "fp8", x["cV_scale"])
    O, lse = sparse_attn(q, cK, cV, idx, decode_kv(x["Kw"], io), decode_kv(x["Vw"], io), raw0, pos, W)
    _run_all_forms(csa, False, x, io, None, idx, raw0, pos, W, B, T, H, O, lse)


def test_chain_compress_fp8_then_dense(csa):
    """Raw bf16 K/V (with outliers) -> csa_compress_kv (fp8, m' = 128) -> hca_dense_attn, against
    the oracle's pool, E4M3 storage and attention on the same raw K/V."""
    B, mp, n_ent, W, H = 2, 128, 160, 128, 64
    L = mp * n_ent
    say(f"fp8 chain: compress m'={mp} ({n_ent} entries) then dense attention, B={B}")
    kv = compress_inputs(B, L, "bf16", seed=5, tag=72, outliers=True)
    K64, V64 = bf16_decode(kv["K"]), bf16_decode(kv["V"])
    Kh, Vh = compress_values(K64, V64, kv["logits"], mp)
    (ck_o, cks_o), (cv_o, cvs_o) = store(Kh, "fp8"), store(Vh, "fp8")
    pos = np.array([L - 1, L - 1 - 3 * mp], np.int32)
    raw0 = (pos + 1 - W).astype(np.int32)
    q = normal_kv(streams(73, 0, 1)[0], (B, 1, H, D), "bf16")
    win = (raw0[:, None] + np.arange(W)[None]).astype(np.int64)
    Kw = np.stack([kv["K"][b, win[b]] for b in range(B)])
    Vw = np.stack([kv["V"][b, win[b]] for b in range(B)])
    O, lse = dense_attn(bf16_decode(q), decode_kv(ck_o, "fp8", cks_o), decode_kv(cv_o, "fp8", cvs_o), mp,
                        bf16_decode(Kw), bf16_decode(Vw), raw0, pos, W)

    ck = torch.empty((B, n_ent, D), dtype=torch.uint8, device="cuda")
    cv = torch.empty_like(ck)
    cks = torch.empty((B, n_ent), device="cuda")
    cvs = torch.empty_like(cks)
    csa.csa_compress_kv(t_kv(kv["K"], "bf16"), t_kv(kv["V"], "bf16"), t_f32(kv["logits"]), mp, ck, cv, cks, cvs)
    torch.cuda.synchronize()
    g_scale = h(cks).astype(np.float64)
    assert np.any(np.log2(g_scale) % 1 != 0)
    qd, kw, vw = t_kv(q, "bf16"), t_kv(Kw, "bf16"), t_kv(Vw, "bf16")
    for form in ("plain", "batch_invariant"):
        lse_g = torch.empty((B, 1, H), device="cuda")
        out = csa.hca_dense_attn(qd, ck, cv, mp, kw, vw, t_i32(raw0), t_i32(pos), W, ck_scale=cks,
                                 cv_scale=cvs, lse=lse_g, batch_invariant=form != "plain")
        torch.cuda.synchronize()
        _check(form, out, lse_g, O, lse, "bf16")


def test_chain_cache_append_fp8_then_sparse(csa):
    """A run of csa_kv_cache_append calls (m = 4, fp8 entries, one sequence idling at times)
    fills a cache that csa_sparse_attn then reads through the ring; the oracle pools the same
    tokens, stores with its E4M3 rule and attends over the linear history.  (bf16 I/O only: a
    one-unit E4M3 flip between two independently pooled caches moves an output by about
    1e-3, inside 2e-2 but not inside the fp32 bound; fp32 I/O is checked on identical caches
    above.)"""
    io = "bf16"
    B, m, L, cap, steps, H, k = 3, 4, 128, 256, 1000, 64, 128
    W = L
    say(f"fp8 chain: {steps} cache appends (m={m}, io={io}) then sparse attention, B={B}")
    n_total = steps + m
    x = compress_inputs(B, n_total, io, seed=6, tag=74, outliers=True)
    Kd, Vd, Zd = t_kv(x["K"], io), t_kv(x["V"], io), t_f32(x["logits"])
    ring_k = torch.zeros((B, 2 * L, D), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    ring_z = torch.zeros((B, 2 * L), device="cuda")
    ck = torch.zeros((B, cap, D), dtype=torch.uint8, device="cuda")
    cv = torch.zeros_like(ck)
    cks = torch.ones((B, cap), device="cuda")
    cvs = torch.ones_like(cks)
    nxt = np.zeros(B, np.int64)
    ar = torch.arange(B, device="cuda")
    raw0 = None
    for s in range(steps):
        active = np.array([not (b == 1 and s % 5 == 2) for b in range(B)])
        pos = np.where(active, nxt, -1).astype(np.int32)
        pd = t_i32(pos)
        src = pd.long().clamp(min=0)
        raw0 = csa.csa_kv_cache_append(Kd[ar, src].contiguous(), Vd[ar, src].contiguous(), Zd[ar, src].contiguous(),
                                       pd, ring_k, ring_v, ring_z, m, ck, cv, ck_scale=cks, cv_scale=cvs)
        nxt += active
    torch.cuda.synchronize()
    last = (nxt - 1).astype(np.int32)

    Kx, Vx = bf16_decode(x["K"]), bf16_decode(x["V"])
    Kh, Vh = compress_values(Kx, Vx, x["logits"], m)
    (ck_o, cks_o), (cv_o, cvs_o) = store(Kh, "fp8"), store(Vh, "fp8")
    cK_o = decode_kv(ck_o, "fp8", cks_o)
    cV_o = decode_kv(cv_o, "fp8", cvs_o)
    nv = np.minimum(nvis(last[:, None], m), cap)
    assert np.all(nv == np.array([int(n) // m for n in nxt])[:, None])
    idx = random_topk_idx(nv, k, cap, seed=7)
    q = normal_kv(streams(75, 0, 1)[0], (B, 1, H, D), io)
    zero = np.zeros(B, np.int32)
    O, lse = sparse_attn(decode_kv(q, io), cK_o, cV_o, idx, Kx, Vx, zero, last, W)
    qd = t_kv(q, io)
    for form in ("plain", "batch_invariant"):
        lse_g = torch.empty((B, 1, H), device="cuda")
        out = csa.csa_sparse_attn(qd, ck, cv, t_i32(idx), ring_k, ring_v, raw0, t_i32(last), W, ck_scale=cks,
                                  cv_scale=cvs, lse=lse_g, batch_invariant=form != "plain")
        torch.cuda.synchronize()
        _check(form, out, lse_g, O, lse, io)


def test_dense_many_query_scale_swings(csa):
    """The many-query dense kernel (plain call, >= 256 query rows) over fp8 entries whose V
    scales swing across chunks of 64 entries: 2^20 (with keys pointing away from every query,
    so their weights are ~2^-70 and their products vanish), 2^-12, and 1 elsewhere.  The kernel
    carries its output in units of a power-of-two V-scale reference that must follow the scales
    down again after a large chunk, or the fp16 P of the following chunks would fall into
    fp16's subnormal range; the check is the usual element-wise one against the oracle."""
    from csa_synth.gen import f32_to_bf16_bits
    io, B, T, H, mp, cap, W = "bf16", 1, 256, 64, 16, 1024, 64
    say(f"fp8 V-scale swings: dense many-query T={T} H={H} m'={mp} cap={cap} W={W}")
    pos = np.array([cap * mp - T], np.int32)   # the last query sees all cap entries
    L_raw = T + W
    raw0 = (pos + T - L_raw).astype(np.int32)
    rq, rk, rv, rkw, rvw, ru = streams(75, 0, 6)
    u = ru.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    q = f32_to_bf16_bits(normal_f32(rq, (B, T, H, D)) + 8.0 * u)
    factor = np.ones(cap // 64, np.float32)
    far = np.zeros(cap // 64, bool)
    factor[[1, 7]] = 2.0 ** 20
    far[[1, 7]] = True
    factor[6] = 2.0 ** -12
    Kt = normal_f32(rk, (B, cap, D))
    Kt[:, np.repeat(far, 64)] = -200.0 * u
    Vt = normal_f32(rv, (B, cap, D)) * np.repeat(factor, 64)[None, :, None]
    cK, cKs = store(Kt.astype(np.float64), "fp8")
    cV, cVs = store(Vt.astype(np.float64), "fp8")
    Kw, Vw = normal_kv(rkw, (B, L_raw, D), io), normal_kv(rvw, (B, L_raw, D), io)
    O, lse = dense_attn(decode_kv(q, io), decode_kv(cK, "fp8", cKs), decode_kv(cV, "fp8", cVs), mp,
                        decode_kv(Kw, io), decode_kv(Vw, io), raw0, pos, W)
    assert np.abs(O).max() < 20.0   # the far chunks' products do vanish
    x = dict(q=q, cK=cK, cK_scale=cKs, cV=cV, cV_scale=cVs, Kw=Kw, Vw=Vw)
    _run_all_forms(csa, True, x, io, mp, None, raw0, pos, W, B, T, H, O, lse)
