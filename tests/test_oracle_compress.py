"""Pins of the oracle's softmax-pool compression (closed forms, invariants, brute force)."""
import os
from fractions import Fraction

import numpy as np
import torch

from csa_synth import compress_inputs
from oracle import brute
from oracle.compress import compress_kv, compress_values, fp8_quantize_entries, pool_weights
from oracle.formats import bf16_decode, e4m3_decode, e4m3_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(B, L, seed=0):
    x = compress_inputs(B, L, seed=seed)
    return bf16_decode(x["K"]), bf16_decode(x["V"]), x["logits"].astype(np.float64), x


def test_count_shrinks_by_m():
    for line in open(os.path.join(GOLDEN, "compression_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        L, m, exp = map(int, line.split())
        assert L // m == exp
    K, V, z, _ = _kv(2, 37)
    for m in (1, 2, 4, 5, 8, 37):
        Kh, Vh = compress_values(K, V, z, m)
        assert Kh.shape == (2, 37 // m, 128) and Vh.shape == Kh.shape


def test_m1_is_identity_bit_exact():
    K, V, z, raw = _kv(2, 16)
    (kb, vb) = compress_kv(K, V, z, 1, "bf16")
    assert np.array_equal(kb, raw["K"]) and np.array_equal(vb, raw["V"])


def test_equal_logits_give_the_arithmetic_mean():
    K, V, _, _ = _kv(1, 32)
    z = np.zeros((1, 32))
    Kh, _ = compress_values(K, V, z, 4)
    # exact rational mean of the 4 bf16 values in each block
    for e in range(8):
        for c in (0, 17, 127):
            mean = sum(Fraction(float(K[0, 4 * e + j, c])) for j in range(4)) / 4
            assert Fraction(float(Kh[0, e, c])) == mean


def test_dominant_logit_selects_one_token():
    K, V, _, _ = _kv(1, 8)
    z = np.full((1, 8), -100.0)
    z[0, 0] = 0.0
    z[0, 6] = 0.0
    Kh, Vh = compress_values(K, V, z, 4)
    assert np.abs(Kh[0, 0] - K[0, 0]).max() < 1e-40
    assert np.abs(Vh[0, 1] - V[0, 6]).max() < 1e-40


def test_convexity_and_weights_sum_to_one():
    K, V, z, _ = _kv(3, 64, seed=3)
    for m in (2, 4, 16):
        a = pool_weights(z.reshape(3, -1, m))
        assert np.allclose(a.sum(-1), 1.0, atol=1e-15, rtol=0)
        assert np.all(a > 0)
        Kh, _ = compress_values(K, V, z, m)
        blocks = K.reshape(3, -1, m, 128)
        assert np.all(Kh >= blocks.min(2) - 1e-12) and np.all(Kh <= blocks.max(2) + 1e-12)


def test_pool_weights_match_torch_softmax():
    z = np.random.default_rng(1).standard_normal((50, 128)) * 5
    ref = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
    assert np.abs(pool_weights(z) - ref).max() < 1e-15


def test_fp8_entry_quantisation():
    r = np.random.default_rng(2)
    X = r.standard_normal((40, 128)) * np.exp2(r.integers(-8, 8, (40, 1)))
    X[0] = 0.0
    codes, scale = fp8_quantize_entries(X)
    assert scale[0] == 1.0 and np.all(e4m3_decode(codes[0]) == 0)
    deq = e4m3_decode(codes) * scale[:, None].astype(np.float64)
    amax = np.abs(X[1:]).max(1)
    # scale is the fp32 rounding of amax / 448
    assert np.array_equal(scale[1:], (amax / 448.0).astype(np.float32))
    # every code is the RNE E4M3 value of x / scale (within the format's half-ulp)
    y = X / scale[:, None].astype(np.float64)
    assert np.array_equal(e4m3_decode(codes), e4m3_round(y))
    # the largest-magnitude element of each entry lands at (about) +-448
    i = np.abs(X[1:]).argmax(1)
    top = np.abs(e4m3_decode(codes[1:])[np.arange(39), i])
    assert np.all((top == 448.0) | (top == 416.0))
    err = np.abs(deq - X)[1:]
    assert np.all(err <= 2.0 ** -4 * np.abs(X[1:]) + 2.0 ** -10 * scale[1:, None])


def test_matches_pure_python_brute_force():
    K, V, z, _ = _kv(2, 12, seed=5)
    K, V = K[:, :, :6], V[:, :, :6]
    for m in (1, 2, 3, 4):
        Kh, Vh = compress_values(K, V, z, m)
        bk, bv = brute.compress(K.tolist(), V.tolist(), z.tolist(), m)
        assert np.abs(Kh - np.array(bk)).max() < 1e-14
        assert np.abs(Vh - np.array(bv)).max() < 1e-14
