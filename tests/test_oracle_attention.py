"""Pins of the oracle's CSA sparse / HCA dense attention."""
import math

import numpy as np
import torch

from csa_synth import attn_inputs, random_topk_idx
from oracle import brute
from oracle.attention import decode_kv, dense_attn, layer_pair, sparse_attn
from oracle.formats import bf16_decode


def _seq(n, H, seed):
    """One sequence of n raw tokens (K, V) and n queries, fp64 values of bf16 draws."""
    x = attn_inputs(1, n, H, n, n, seed=seed)
    return bf16_decode(x["q"]), bf16_decode(x["Kw"]), bf16_decode(x["Vw"])


def _sdpa(q, K, V, mask=None):
    """torch CPU fp64 scaled_dot_product_attention, causal, all heads share K/V."""
    qt = torch.from_numpy(q[0]).permute(1, 0, 2)                # [H, T, d]
    H = qt.shape[0]
    kt = torch.from_numpy(K[0])[None].expand(H, -1, -1)
    vt = torch.from_numpy(V[0])[None].expand(H, -1, -1)
    if mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()[None]


def test_csa_m1_all_entries_no_window_is_full_causal_attention():
    n, H = 40, 4
    q, K, V = _seq(n, H, seed=1)
    # m = 1: every token is its own compressed entry (pool of one = the token itself)
    idx = np.full((1, n, n), -1, np.int32)
    for t in range(n):
        idx[0, t, : t + 1] = np.arange(t + 1)
    O, _ = sparse_attn(q, K, V, idx, K, V, np.array([0]), np.array([0]), W=0)
    assert np.abs(O - _sdpa(q, K, V)).max() < 1e-12


def test_csa_m1_all_entries_with_window_closed_form():
    """Window keys appear twice (entry + raw token): logit + ln 2 on the last W keys."""
    n, H, W = 33, 2, 5
    q, K, V = _seq(n, H, seed=2)
    idx = np.full((1, n, n), -1, np.int32)
    for t in range(n):
        idx[0, t, : t + 1] = np.arange(t + 1)
    O, _ = sparse_attn(q, K, V, idx, K, V, np.array([0]), np.array([0]), W=W)
    mask = torch.full((n, n), -math.inf, dtype=torch.float64)
    for t in range(n):
        mask[t, : t + 1] = 0.0
        mask[t, max(0, t - W + 1): t + 1] = math.log(2.0)
    assert np.abs(O - _sdpa(q, K, V, mask)).max() < 1e-12


def test_hca_m1_no_window_is_full_causal_attention():
    n, H = 37, 3
    q, K, V = _seq(n, H, seed=3)
    O, _ = dense_attn(q, K, V, 1, K, V, np.array([0]), np.array([0]), W=0)
    assert np.abs(O - _sdpa(q, K, V)).max() < 1e-12


def test_invariants():
    B, T, H, cap, W = 2, 3, 4, 50, 6
    x = attn_inputs(B, T, H, cap, 20, seed=4)
    q = bf16_decode(x["q"])
    cK, cV = bf16_decode(x["cK"]), bf16_decode(x["cV"])
    Kw = bf16_decode(x["Kw"])
    pos0 = np.array([100, 150])
    raw0 = pos0 + T - 20
    nv = np.stack([(pos0[b] + np.arange(T) + 1) // 4 for b in range(B)])
    idx = random_topk_idx(nv, 9, cap, seed=4)
    ones = np.ones_like(cV)
    O, lse = sparse_attn(q, cK, ones, idx, Kw, np.ones_like(Kw), raw0, pos0, W)
    assert np.abs(O - 1.0).max() < 1e-12                       # rows of p sum to 1
    # constant V rows -> that constant
    O, _ = sparse_attn(q, cK, 3.5 * ones, idx, Kw, 3.5 * np.ones_like(Kw), raw0, pos0, W)
    assert np.abs(O - 3.5).max() < 1e-12
    # invariance to permuting the idx list
    O1, l1 = sparse_attn(q, cK, cV, idx, Kw, bf16_decode(x["Vw"]), raw0, pos0, W)
    O2, l2 = sparse_attn(q, cK, cV, idx[..., ::-1].copy(), Kw, bf16_decode(x["Vw"]), raw0, pos0, W)
    assert np.abs(O1 - O2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
    # a single key -> O = its value, lse = its logit
    one = np.full((1, 1, 1), -1, np.int32)
    one[0, 0, 0] = 7
    O, lse = sparse_attn(q[:1, :1], cK, cV, one, Kw, Kw, raw0, pos0, 0)
    assert np.abs(O[0, 0] - cV[0, 7][None]).max() < 1e-15
    assert np.abs(lse[0, 0] - q[0, 0] @ cK[0, 7] / math.sqrt(128)).max() < 1e-12


def test_empty_key_set():
    x = attn_inputs(1, 1, 2, 4, 4, seed=5)
    q = bf16_decode(x["q"])
    cK = bf16_decode(x["cK"])
    idx = np.full((1, 1, 3), -1, np.int32)
    O, lse = sparse_attn(q, cK, cK, idx, cK, cK, np.array([0]), np.array([2]), 0)
    assert np.all(O == 0) and np.all(lse == -np.inf)
    O, lse = dense_attn(q, cK, cK, 4, cK, cK, np.array([0]), np.array([2]), 0)
    assert np.all(O == 0) and np.all(lse == -np.inf)


def test_fp8_entries_decode_as_code_times_scale():
    x = attn_inputs(1, 1, 1, 8, 4, ckv_dtype="fp8", seed=6)
    v = decode_kv(x["cK"], "fp8", x["cK_scale"])
    ref = torch.from_numpy(x["cK"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v, ref * x["cK_scale"][..., None].astype(np.float64))


def test_brute_force_small():
    r = np.random.default_rng(7)
    for trial in range(6):
        m = int(r.choice([1, 2, 4]))
        W = int(r.choice([0, 3, 8]))
        B, T, H, cap = 1, 2, 2, 12
        n = cap * m
        pos0 = np.array([n - T])
        L_raw = 10
        raw0 = np.array([n - L_raw])
        x = attn_inputs(B, T, H, cap, L_raw, seed=10 + trial)
        q = bf16_decode(x["q"])[..., :8]
        cK, cV = bf16_decode(x["cK"])[..., :8], bf16_decode(x["cV"])[..., :8]
        Kw, Vw = bf16_decode(x["Kw"])[..., :8], bf16_decode(x["Vw"])[..., :8]
        nv = (pos0[0] + np.arange(T) + 1)[None] // m
        for k in (1, 3, cap):
            idx = random_topk_idx(nv, k, cap, seed=trial)
            sm = 1 / math.sqrt(8)
            O, lse = sparse_attn(q, cK, cV, idx, Kw, Vw, raw0, pos0, W, sm)
            for i in range(T):
                bo, bl = brute.csa_attend(q[0, i].tolist(), cK[0].tolist(), cV[0].tolist(),
                                          idx[0, i].tolist(), Kw[0].tolist(), Vw[0].tolist(),
                                          int(raw0[0]), int(pos0[0]) + i, W, sm)
                assert np.abs(O[0, i] - np.array(bo)).max() < 1e-12
                assert np.abs(lse[0, i] - np.array(bl)).max() < 1e-12
        O, lse = dense_attn(q, cK, cV, m, Kw, Vw, raw0, pos0, W, 1 / math.sqrt(8))
        for i in range(T):
            bo, bl = brute.hca_attend(q[0, i].tolist(), cK[0].tolist(), cV[0].tolist(), m,
                                      Kw[0].tolist(), Vw[0].tolist(), int(raw0[0]),
                                      int(pos0[0]) + i, W, 1 / math.sqrt(8))
            assert np.abs(O[0, i] - np.array(bo)).max() < 1e-12


def test_layer_pair_is_the_two_calls():
    x = attn_inputs(1, 1, 2, 8, 8, seed=8)
    q = bf16_decode(x["q"])
    c = bf16_decode(x["cK"])
    kw = dict(q=q, cK=c, cV=c, Kw=c, Vw=c, raw_pos0=np.array([24]), q_pos0=np.array([31]), W=4)
    idx = np.array([[[0, 3, -1]]], np.int32)
    (o1, _), (o2, _) = layer_pair(dict(kw, idx=idx), dict(kw, m_prime=4))
    assert np.array_equal(o1, sparse_attn(idx=idx, **kw)[0])
    assert np.array_equal(o2, dense_attn(m_prime=4, **kw)[0])
