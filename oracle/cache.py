"""Decode-time KV cache with a mirrored window ring (test infrastructure).

This module is the oracle of the cache append; only the tests, the smoke check and the
benchmark's CPU baseline use it.

Pages: the newest uncompressed tokens (the sliding window) are kept in bf16 next to the
compressed entries, which may be stored in fp8 (the ferris DeepSeek-V4 analysis, 工程层,
heterogeneous KV cache); every m tokens' K/V become one entry (blog.nickys.cn DeepSeek-V4
post, 三大架构改动 §1 CSA, §2 HCA).

Readings (the pages give no cache layout; these are the library's definitions):
  * A sequence's window lives in 2L rows.  Appending token p writes it to rows p mod L and
    p mod L + L.
  * After tokens 0 .. n-1 were appended in order, row r holds the latest token p < n with
    p = r (mod L), or nothing if there is none (ring_rows below).
  * A query at position p reads its window through a raw buffer of 2L rows whose row 0
    stands for position window_base(p, L) = q0 - (q0 mod L), q0 = max(0, p - L + 1).
  * When token p completes a block (p + 1 = 0 mod m), entry (p + 1)/m - 1 becomes the pool
    of tokens p - m + 1 .. p (oracle.compress).  That is the same entry the compression of
    the whole linear history gives.  Entries at or past the cache's capacity are dropped.
"""
import numpy as np


def append_step_by_step(X, n, L, start=0):
    """The 2L ring rows after appending tokens start .. n-1 of history X [n_total, ...] one at
    a time, each written to rows p mod L and p mod L + L.  Returns (rows, written mask)."""
    rows = np.zeros((2 * L,) + X.shape[1:], X.dtype)
    written = np.zeros(2 * L, bool)
    for p in range(start, n):
        for r in (p % L, p % L + L):
            rows[r] = X[p]
            written[r] = True
    return rows, written


def ring_rows(X, n, L, start=0):
    """Closed form of the same state: row r holds the largest p in [start, n) with
    p = r (mod L)."""
    rows = np.zeros((2 * L,) + X.shape[1:], X.dtype)
    written = np.zeros(2 * L, bool)
    for r in range(2 * L):
        res = r % L
        if n - 1 < start:
            continue
        p = (n - 1) - ((n - 1 - res) % L)      # largest p <= n - 1 with p = res (mod L)
        if p >= start:
            rows[r] = X[p]
            written[r] = True
    return rows, written


def window_base(p, L):
    """Position that row 0 of the 2L-row ring stands for when a query at p reads it."""
    if p < 0:
        return 0
    q0 = max(0, p - L + 1)
    return q0 - q0 % L


def appended_entries(n, m, cap, start=0):
    """Indices of the entries that appending tokens start .. n-1 writes (start a multiple of
    m): the blocks completed by those tokens, below the capacity."""
    return [e for e in range(start // m, n // m) if e < cap]
