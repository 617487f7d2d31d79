"""Pins of the oracle's top-k selection (library sort, invariants, ties, brute force)."""
import numpy as np

from csa_synth import indexer_inputs, random_scores
from oracle import brute
from oracle.indexer import indexer_scores, nvis
from oracle.topk import topk, topk_row


def _check_invariants(row, nv, k, out):
    sel = out[out >= 0]
    assert np.all(np.diff(sel) > 0)                       # ascending, distinct
    assert sel.size == min(k, nv) and np.all(out[sel.size:] == -1)
    assert np.all(sel < nv)
    if sel.size < nv:
        rest = np.setdiff1d(np.arange(nv), sel)
        lo = row[sel].min()
        hi = row[rest].max()
        assert lo >= hi                                   # every selected >= every unselected
        if lo == hi:                                      # boundary ties: lowest indices taken
            tied_sel = sel[row[sel] == lo]
            tied_rest = rest[row[rest] == hi]
            assert tied_sel.max() < tied_rest.min()


def test_matches_stable_argsort_and_invariants():
    s = random_scores(3, 4, 300, seed=1, distinct=40).astype(np.float64)
    for b in range(3):
        for i in range(4):
            for nv, k in ((300, 17), (300, 300), (123, 64), (5, 64), (0, 8)):
                out = topk_row(s[b, i], nv, k)
                ref = np.sort(np.argsort(-s[b, i, :nv], kind="stable")[:k])
                assert np.array_equal(out[: ref.size], ref)
                _check_invariants(s[b, i], nv, k, out)


def test_signed_zero_is_one_value():
    row = np.array([-0.0, 0.0, -0.0, 1.0, 0.0, -1.0])
    assert topk_row(row, 6, 3).tolist() == [0, 1, 3]
    assert topk_row(row, 6, 4).tolist() == [0, 1, 2, 3]


def test_tie_heavy_indexer_scores_against_brute_force():
    # codes in {0, +-1}, scales 2^0, w = 1: small integer scores, many boundary ties
    B, T, cap, H, dI, m, k = 1, 2, 1024, 4, 64, 4, 64
    x = indexer_inputs(B, T, cap, H, dI, seed=3, tie_heavy=True)
    pos = np.array([cap * m - T])
    s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"], pos, m)
    out = topk(s.astype(np.float32), pos, m, k)
    ties_seen = 0
    for i in range(T):
        t = int(pos[0]) + i
        ref = brute.topk(s[0, i].tolist(), t, m, k)
        assert out[0, i].tolist() == ref
        nv = int(nvis(t, m))
        kth = np.sort(s[0, i, :nv])[::-1][k - 1]
        ties_seen = max(ties_seen, int(np.sum(s[0, i, :nv] == kth)))
        _check_invariants(s[0, i], nv, k, out[0, i])
    assert ties_seen > 3


def test_all_zero_row_takes_lowest_indices():
    s = np.zeros((1, 1, 50), np.float32)
    s[0, 0, ::3] = -0.0
    out = topk(s, np.array([199]), 4, 10)
    assert out[0, 0].tolist() == list(range(10))


def test_brute_force_small_random():
    r = np.random.default_rng(5)
    for trial in range(30):
        cap = int(r.integers(1, 40))
        m = int(r.choice([1, 2, 4]))
        k = int(r.integers(1, 12))
        t = int(r.integers(0, cap * m))
        row = r.integers(-3, 4, cap).astype(np.float64)
        nv = (t + 1) // m
        assert topk_row(row, nv, k).tolist() == brute.topk(row.tolist(), t, m, k)
