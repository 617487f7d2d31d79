"""GPU parity of the combined compression + indexer top-k call (csa_compress_indexer_topk).

The call promises exactly the results of csa_compress_kv followed by
csa_indexer_topk.  Checked here: idx against the oracle (indexer scores, then
top-k with the lower-index tie rule), bit for bit; the compressed entries
against the oracle pool within one storage unit, and bit for bit against the
separate csa_compress_kv call; slots outside the pooled range untouched.
Cases cover the decoding shapes where the compression rides in the
selection's launch (one and several compression blocks, every storage type,
fp32 inputs, a row with fewer visible entries than k) and a prefill chunk,
where the two run as separate launches; bad arguments of either part are
rejected before anything runs.
"""
import numpy as np
import pytest
import torch

from csa_synth import compress_inputs, indexer_inputs
from gpu_helpers import compress_tolerance, h, h_bf16, say, t_f32, t_i32, t_kv, t_u8
from oracle.compress import compress_values, store
from oracle.formats import bf16_decode, e4m3_decode
from oracle.indexer import indexer_scores
from oracle.topk import topk

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _kv64(x, dt):
    return bf16_decode(x) if dt == "bf16" else np.asarray(x, np.float64)


def _outputs(B, n_slots, out_dt):
    ko = torch.full((B, n_slots, 128), 7, dtype=TDT[out_dt], device="cuda")
    vo = torch.full((B, n_slots, 128), 7, dtype=TDT[out_dt], device="cuda")
    ks = vs = None
    if out_dt == "fp8":
        ks = torch.full((B, n_slots), -1.0, device="cuda")
        vs = torch.full((B, n_slots), -1.0, device="cuda")
    return ko, vo, ks, vs


def _check_pool(x, in_dt, out_dt, m, row0, L, entry0, outs):
    """Entries entry0 .. entry0 + L/m - 1 against the oracle pool of rows row0 .. row0 + L - 1."""
    ko, vo, ks, vs = outs
    n = L // m
    K = _kv64(x["K"], in_dt)[:, row0:row0 + L]
    V = _kv64(x["V"], in_dt)[:, row0:row0 + L]
    Kh, Vh = compress_values(K, V, x["logits"][:, row0:row0 + L], m)
    B = K.shape[0]
    amax = np.abs(np.stack([K, V])).reshape(2, B, n, m, 128).max(axis=(3, 4))
    sl = slice(entry0, entry0 + n)
    for which, X, out, sc in ((0, Kh, ko, ks), (1, Vh, vo, vs)):
        eps = (m + 4) * 2.0 ** -24 * amax[which][..., None]
        if out_dt == "bf16":
            g, o = bf16_decode(h_bf16(out))[:, sl], bf16_decode(store(X, "bf16"))
            tol = compress_tolerance(X, "bf16", eps)
        elif out_dt == "f32":
            g, o = h(out).astype(np.float64)[:, sl], store(X, "f32").astype(np.float64)
            tol = compress_tolerance(X, "f32", eps)
        else:
            codes, scale = store(X, "fp8")
            g = e4m3_decode(h(out))[:, sl] * h(sc).astype(np.float64)[:, sl, None]
            o = e4m3_decode(codes) * scale[..., None].astype(np.float64)
            tol = compress_tolerance(X, "fp8", eps, scale)
        assert np.all(np.abs(g - o) <= tol), np.abs(g - o).max()
        rest = torch.ones(out.shape[1], dtype=torch.bool)
        rest[sl] = False
        assert torch.equal(out[:, rest], torch.full_like(out[:, rest], 7))


CASES = [
    # B, T, cap, H_I, d_I, m, k, pos0 list, L_raw, L, in, out
    (3, 1, 32768, 8, 128, 4, 1024, [131071, 100000, 2000], 64, 4, "bf16", "bf16"),  # 128K decode rows
    (2, 1, 9000, 4, 64, 4, 300, [35999, 20000], 64, 4, "bf16", "fp8"),             # fp8 entries
    (2, 1, 10000, 16, 256, 2, 500, [19999, 15000], 40, 2, "f32", "f32"),          # fp32 in, m = 2
    (2, 1, 12000, 8, 128, 4, 700, [47999, 40000], 1400, 1200, "bf16", "bf16"),    # 600 entries: 10 blocks
    (1, 6, 20000, 8, 128, 4, 500, [79990], 48, 24, "bf16", "f32"),               # prefill chunk: two launches
]


@pytest.mark.parametrize("B,T,cap,H_I,d_I,m,k,pos,L_raw,L,in_dt,out_dt", CASES)
def test_combined_matches_oracle_and_separate_calls(csa, B, T, cap, H_I, d_I, m, k, pos, L_raw, L,
                                                     in_dt, out_dt):
    say(f"compress_indexer_topk B={B} T={T} cap={cap} H_I={H_I} k={k} L={L} {in_dt}->{out_dt}")
    xi = indexer_inputs(B, T, cap, H_I, d_I, seed=cap + k)
    xc = compress_inputs(B, L_raw, in_dt, seed=L + B)
    pos = np.array(pos, np.int32)
    row0 = L_raw - L
    n_slots = L // m + 5
    entry0 = 3
    kin, vin, lg = t_kv(xc["K"], in_dt), t_kv(xc["V"], in_dt), t_f32(xc["logits"])
    dev_ix = (t_u8(xi["q_codes"]), t_u8(xi["q_e8m0"]), t_f32(xi["w"]), t_u8(xi["k_codes"]),
              t_u8(xi["k_e8m0"]), t_i32(pos))

    outs = _outputs(B, n_slots, out_dt)
    idx = csa.csa_compress_indexer_topk(kin, vin, lg, *outs, *dev_ix, m, k, L=L, row0=row0,
                                        entry0=entry0)
    sep = _outputs(B, n_slots, out_dt)
    csa.csa_compress_kv(kin, vin, lg, m, *sep, L=L, row0=row0, entry0=entry0)
    torch.cuda.synchronize()

    s = indexer_scores(xi["q_codes"], xi["q_e8m0"], xi["w"], xi["k_codes"], xi["k_e8m0"], pos, m)
    ref = topk(s.astype(np.float32), pos, m, k)
    got = h(idx)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
    for a, b in zip(outs, sep):
        if a is not None:
            assert torch.equal(a, b)
    _check_pool(xc, in_dt, out_dt, m, row0, L, entry0, outs)


def test_combined_rejects_bad_arguments_before_running(csa):
    """A bad compression argument (m not dividing L) or a bad indexer argument (H_I = 5)
    fails the call and leaves every output untouched."""
    say("compress_indexer_topk argument errors")
    B, cap, H_I, d_I, m, k = 2, 9000, 4, 64, 4, 300
    xi = indexer_inputs(B, 1, cap, H_I, d_I, seed=5)
    xc = compress_inputs(B, 16, "bf16", seed=6)
    pos = np.array([35999, 20000], np.int32)
    kin, vin, lg = t_kv(xc["K"], "bf16"), t_kv(xc["V"], "bf16"), t_f32(xc["logits"])
    outs = _outputs(B, 8, "bf16")
    idx = torch.full((B, 1, k), -7, dtype=torch.int32, device="cuda")
    dev_ix = [t_u8(xi["q_codes"]), t_u8(xi["q_e8m0"]), t_f32(xi["w"]), t_u8(xi["k_codes"]),
              t_u8(xi["k_e8m0"]), t_i32(pos)]
    with pytest.raises(RuntimeError):
        csa.csa_compress_indexer_topk(kin, vin, lg, *outs, *dev_ix, m, k, idx=idx, L=6, row0=0)
    bad_q = t_u8(np.zeros((B, 1, 5, d_I // 2), np.uint8))
    bad_e = t_u8(np.full((B, 1, 5, d_I // 32), 127, np.uint8))
    bad_w = t_f32(np.ones((B, 1, 5), np.float32))
    with pytest.raises(RuntimeError):
        csa.csa_compress_indexer_topk(kin, vin, lg, *outs, bad_q, bad_e, bad_w, *dev_ix[3:], m, k,
                                      idx=idx, L=4, row0=12)
    torch.cuda.synchronize()
    for t in outs:
        if t is not None:
            assert torch.equal(t, torch.full_like(t, 7))
    assert torch.equal(idx, torch.full_like(idx, -7))
