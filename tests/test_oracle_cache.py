"""Pins of the cache oracle (oracle/cache.py).

The closed form of the ring state is checked against the step-by-step write sequence. The
window read through window_base is checked, by brute force on small sizes, to return every
token of every window W <= L, for every query position. A wrong modulus, a wrong copy
offset or an off-by-one in q0 fails these.
"""
import numpy as np

from oracle.cache import append_step_by_step, appended_entries, ring_rows, window_base


def test_closed_form_matches_step_by_step():
    X = np.arange(1, 200 * 3 + 1).reshape(200, 3)
    for L in (1, 2, 5, 8, 16):
        for start in (0, 3, 16):
            for n in range(start, 60):
                a, wa = ring_rows(X, n, L, start)
                b, wb = append_step_by_step(X, n, L, start)
                assert np.array_equal(wa, wb), (L, start, n)
                assert np.array_equal(a[wa], b[wb]), (L, start, n)


def test_window_through_the_ring_is_the_window():
    X = np.arange(1000)
    for L in (1, 3, 4, 8, 13):
        for p in range(0, 80):
            rows, written = ring_rows(X, p + 1, L)
            base = window_base(p, L)
            for W in range(1, L + 1):
                for q in range(max(0, p - W + 1), p + 1):
                    r = q - base
                    assert 0 <= r < 2 * L and written[r] and rows[r] == q, (L, p, W, q)
            # no row of the window's run stands for a position past the query
            assert base <= max(0, p - L + 1)
    assert window_base(-1, 8) == 0


def test_appended_entries():
    assert appended_entries(12, 4, 10) == [0, 1, 2]
    assert appended_entries(11, 4, 10) == [0, 1]
    assert appended_entries(40, 4, 5) == [0, 1, 2, 3, 4]
    assert appended_entries(16, 4, 10, start=8) == [2, 3]
    assert appended_entries(3, 4, 10) == []
