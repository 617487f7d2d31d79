"""Pins of the oracle's lightning-indexer scores."""
from fractions import Fraction

import numpy as np
import pytest

from csa_synth import indexer_inputs, mxfp4_random, streams
from oracle import brute
from oracle.indexer import indexer_scores, nvis


def test_exact_rational_recomputation():
    B, T, cap, H, dI, m = 1, 2, 24, 3, 64, 4
    x = indexer_inputs(B, T, cap, H, dI, seed=1)
    q_pos0 = np.array([70])
    s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"], q_pos0, m)
    for i in range(T):
        t = 70 + i
        Q = [[Fraction(v) for v in brute.mxfp4_vector(x["q_codes"][0, i, h], x["q_e8m0"][0, i, h])]
             for h in range(H)]
        for e in range(cap):
            if e >= (t + 1) // m:
                assert s[0, i, e] == -np.inf
                continue
            Kx = [Fraction(v) for v in brute.mxfp4_vector(x["k_codes"][0, e], x["k_e8m0"][0, e])]
            exact = Fraction(0)
            for h in range(H):
                dot = sum(a * b for a, b in zip(Q[h], Kx))
                exact += Fraction(float(x["w"][0, i, h])) * max(dot, Fraction(0))
            assert Fraction(float(s[0, i, e])) == exact
            assert float(np.float32(s[0, i, e])) == s[0, i, e]


def test_integer_matmul_reduction():
    """H_I = 1, w = 1, all scales 2^0: 4*s = ReLU(integer dot of doubled E2M1 codes)."""
    rc, re_ = streams(99, 0, 2)
    B, T, cap, dI = 1, 5, 40, 128
    qc, _ = mxfp4_random(rc, re_, (B, T, 1), dI)
    kc, _ = mxfp4_random(rc, re_, (B, cap), dI)
    qe = np.full((B, T, 1, dI // 32), 127, np.uint8)
    ke = np.full((B, cap, dI // 32), 127, np.uint8)
    w = np.ones((B, T, 1), np.float32)
    pos = np.array([4 * cap - 1 - T])   # nearly every entry visible
    s = indexer_scores(qc, qe, w, kc, ke, pos, 4)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)

    def ints(p):
        return twice[np.stack([p & 15, p >> 4], -1).reshape(p.shape[:-1] + (-1,))]

    qi = ints(qc)[0, :, 0]                       # [T, dI]
    ki = ints(kc)[0]                             # [cap, dI]
    ref = np.maximum(qi @ ki.T, 0)               # int64 matmul
    vis = np.isfinite(s[0])
    assert vis.sum() > 0.9 * vis.size
    assert np.array_equal((4 * s[0])[vis], ref.astype(np.float64)[vis])


def test_generator_bound_keeps_scores_exact():
    """Sum of |terms| stays below 2^24 units of 2^-5 for the generator's ranges."""
    # analytic worst case: 8 heads * w 2 * 128 terms * (6*6 * 2*2)
    worst = 8 * 2 * 128 * 36 * 4
    assert worst * 32 < 2 ** 24
    worst_small = 4 * 2 * 64 * 36 * 4
    assert worst_small * 32 < 2 ** 24
    # the realised inputs at the 128K shapes (sampled rows) are exact as well
    x = indexer_inputs(1, 1, 4096, 8, 128, seed=4)
    s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"],
                       np.array([4096 * 4 - 1]), 4)
    assert np.all(np.isfinite(s)) and np.array_equal(s.astype(np.float32).astype(np.float64), s)


def test_causality_mask():
    x = indexer_inputs(2, 6, 20, 2, 32, seed=2)
    pos = np.array([3, 40])
    s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"], pos, 4)
    for b in range(2):
        for i in range(6):
            nv = min(int(nvis(pos[b] + i, 4)), 20)
            assert np.all(np.isfinite(s[b, i, :nv])) and np.all(s[b, i, nv:] == -np.inf)
    assert nvis(3, 4) == 1 and nvis(2, 4) == 0 and nvis(4095, 4) == 1024


def test_capacity_precondition():
    x = indexer_inputs(1, 1, 4, 1, 32, seed=2)
    with pytest.raises(ValueError):
        indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"],
                       np.array([100]), 4)


def test_matches_pure_python_brute_force():
    B, T, cap, H, dI = 1, 3, 12, 2, 32
    x = indexer_inputs(B, T, cap, H, dI, seed=6)
    for m in (1, 2, 4):
        pos = np.array([cap * m - T])
        s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"], pos, m)
        for i in range(T):
            Q = [brute.mxfp4_vector(x["q_codes"][0, i, h], x["q_e8m0"][0, i, h]) for h in range(H)]
            Kx = [brute.mxfp4_vector(x["k_codes"][0, e], x["k_e8m0"][0, e]) for e in range(cap)]
            ref = brute.indexer(Q, [float(v) for v in x["w"][0, i]], Kx, int(pos[0]) + i, m)
            assert np.array_equal(s[0, i], np.array(ref))
