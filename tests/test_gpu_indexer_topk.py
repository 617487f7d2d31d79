"""GPU parity of the fused indexer + top-k call (csa_indexer_topk).

Against the oracle (indexer scores, then top-k with the lower-index tie rule)
on exact inputs, and bit for bit against the unfused pair of calls
(csa_topk on csa_indexer_scores) on inputs whose scores are NOT exact in fp32,
which the fused call promises to reproduce for any input values.  Cases cover
decode rows, prefill chunks with ragged visibility, rows longer than the part
the kernel keeps in registers, thresholds that fall inside a bucket of exact
ties (including one larger than the on-chip candidate list), and thresholds
that take a whole bucket.
"""
import numpy as np
import pytest
import torch

from csa_synth import indexer_inputs, streams
from gpu_helpers import h, say, t_f32, t_i32, t_u8
from oracle.indexer import indexer_scores
from oracle.topk import topk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import long_context_compressed_03_amd as m
    m.load()
    return m


def _dev(x):
    return (t_u8(x["q_codes"]), t_u8(x["q_e8m0"]), t_f32(x["w"]), t_u8(x["k_codes"]),
            t_u8(x["k_e8m0"]))


def _fused(csa, x, pos, m, k):
    got = csa.csa_indexer_topk(*_dev(x), t_i32(pos), m, k)
    torch.cuda.synchronize()
    return h(got)


FUSED_CASES = [
    # B, T, cap, H_I, d_I, m, k, pos0 list, tie_heavy
    (1, 1, 1024, 4, 64, 4, 64, [4095], False),                     # tiny decode shape
    (3, 1, 32768, 8, 128, 4, 1024, [131071, 100000, 2000], False),  # 128K decode rows; one row < k
    (1, 6, 70000, 8, 128, 4, 2048, [279990], False),               # rows held whole in 20 register rounds
    (1, 3, 90000, 8, 128, 4, 2048, [359990], False),               # rows past the 20-round register chunk
    (1, 3, 70000, 16, 256, 4, 1000, [279990], False),              # d_I = 256: rows past its 16-round chunk
    (2, 33, 5000, 8, 128, 4, 100, [19900, 300], False),            # ragged chunk rows; early rows < k
    (1, 4, 20000, 4, 64, 4, 500, [79990], True),                   # threshold among exact ties
    (1, 3, 3000, 16, 256, 2, 200, [5990], False),                  # 16 heads, two contraction steps
    # decoding rows long enough for the per-slice split path
    (2, 1, 9000, 4, 64, 4, 300, [35999, 20000], False),            # 4 heads, half-width vectors, partial slices
    (2, 1, 10000, 16, 256, 2, 500, [19999, 15000], False),         # 16 heads, two contraction steps
    (1, 1, 16384, 4, 64, 4, 500, [65535], True),                   # exact ties around the threshold
    (1, 1, 100000, 8, 128, 4, 2048, [399999], False),              # 49 slices: 4 per gather wave
    # chunk rows on the threshold path (rows past 32768 entries)
    (1, 3, 50000, 4, 64, 4, 800, [199990], True),                  # exact ties around the threshold
    (2, 9, 45000, 16, 256, 4, 1500, [179990, 150000], False),      # 16 heads, two contraction steps
    (1, 7, 40000, 16, 128, 4, 900, [159990], False),               # 16 heads, one contraction step
    (1, 5, 3000, 16, 128, 4, 300, [11990], False),                 # the same on the 16-bit-key path
]


@pytest.mark.parametrize("B,T,cap,H_I,d_I,m,k,pos,tie", FUSED_CASES)
def test_fused_matches_oracle(csa, B, T, cap, H_I, d_I, m, k, pos, tie):
    say(f"indexer_topk B={B} T={T} cap={cap} H_I={H_I} d_I={d_I} k={k} tie={tie}")
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=cap + k, tie_heavy=tie)
    pos = np.array(pos, np.int32)
    s = indexer_scores(x["q_codes"], x["q_e8m0"], x["w"], x["k_codes"], x["k_e8m0"], pos, m)
    ref = topk(s.astype(np.float32), pos, m, k)
    got = _fused(csa, x, pos, m, k)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_fused_crowded_and_whole_buckets(csa):
    """Row 0: a zero query, so every visible entry ties at score 0 and the threshold
    bucket holds all of them (more than the on-chip list: re-scored in rounds).
    Row 1: exactly k entries score 256 and the rest 0, so the k-th key's bucket is
    taken whole.  Row 2: its own random query against the same keys."""
    say("indexer_topk crowded / whole-bucket rows")
    B, T, cap, H_I, d_I, m, k = 1, 3, 12000, 4, 64, 4, 300
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=77)
    x["q_codes"][0, 0] = 0                                   # row 0: zero query
    x["q_codes"][0, 1] = 0x22                                # row 1: every element +1
    x["q_e8m0"][0, 1] = 127
    x["w"][0, 1] = 1.0
    (r,) = streams(99, 0, 1)
    hot = np.sort(r.choice(cap, size=k, replace=False))
    kc = x["k_codes"].copy()
    ke = x["k_e8m0"].copy()
    kc[0] = 0                                                # keys: zero ...
    kc[0, hot] = 0x22                                        # ... except k of them, all +1
    ke[0] = 127
    x2 = dict(x, k_codes=kc, k_e8m0=ke)
    pos = np.array([4 * cap - 1], np.int32)                 # every row sees all cap entries
    s = indexer_scores(x2["q_codes"], x2["q_e8m0"], x2["w"], kc, ke, pos, m)
    assert np.all(s[0, 0] == 0) and np.sum(s[0, 1] == 256.0) == k
    ref = topk(s.astype(np.float32), pos, m, k)
    assert np.array_equal(ref[0, 0], np.arange(k)) and np.array_equal(ref[0, 1], hot)
    got = _fused(csa, x2, pos, m, k)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_fused_sample_above_the_kth_score(csa):
    """Chunk rows on the threshold path: the sampled entries (the first 16 of every 1024)
    score 256 and the rest 0, so the threshold taken from the sample leaves fewer than k
    entries at or above it; the rows must fall back to the full pass and still select
    exactly (the hot entries, then the lowest-index zeros).  A third row, random, rides
    along, and a fourth has a zero query: every entry ties, more than the candidate
    capacity."""
    say("indexer_topk sample above the k-th score")
    B, T, cap, H_I, d_I, m, k = 1, 4, 40000, 4, 64, 4, 1000
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=79)
    x["q_codes"][0, :2] = 0x22                               # rows 0, 1: every element +1
    x["q_e8m0"][0, :2] = 127
    x["w"][0, :2] = 1.0
    x["q_codes"][0, 3] = 0                                   # row 3: zero query
    kc = x["k_codes"].copy()
    ke = x["k_e8m0"].copy()
    hot = np.array([e for e in range(cap) if e % 1024 < 16])
    kc[0, :] = 0
    kc[0, hot] = 0x22                                        # the sampled entries: +1
    ke[0, :] = 127
    x2 = dict(x, k_codes=kc, k_e8m0=ke)
    pos = np.array([4 * cap - 4], np.int32)
    s = indexer_scores(x2["q_codes"], x2["q_e8m0"], x2["w"], kc, ke, pos, m)
    ref = topk(s.astype(np.float32), pos, m, k)
    assert np.all(np.isin(hot, ref[0, 0])) and np.sum(s[0, 0] == 256.0) == hot.size < k
    assert np.array_equal(ref[0, 3], np.arange(k))
    got = _fused(csa, x2, pos, m, k)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


def test_fused_decode_crowded_rows(csa):
    """Decoding rows on the split path: sequence 0 has a zero query (every entry ties
    at 0: the slice buffers overflow and the row takes the one-block fallback),
    sequence 1 has exactly k entries scoring above the rest (all in a few slices:
    the candidate check fails and the row falls back), sequence 2 is random."""
    say("indexer_topk decode crowded rows")
    B, T, cap, H_I, d_I, m, k = 3, 1, 12000, 4, 64, 4, 300
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=78)
    x["q_codes"][0] = 0
    x["q_codes"][1] = 0x22
    x["q_e8m0"][1] = 127
    x["w"][1] = 1.0
    kc = x["k_codes"].copy()
    ke = x["k_e8m0"].copy()
    kc[1] = 0
    kc[1, 2000:2000 + k] = 0x22                              # k hot entries in one slice
    ke[1] = 127
    x2 = dict(x, k_codes=kc, k_e8m0=ke)
    pos = np.array([4 * cap - 1] * B, np.int32)
    s = indexer_scores(x2["q_codes"], x2["q_e8m0"], x2["w"], kc, ke, pos, m)
    ref = topk(s.astype(np.float32), pos, m, k)
    assert np.array_equal(ref[0, 0], np.arange(k)) and np.array_equal(ref[1, 0], np.arange(2000, 2000 + k))
    got = _fused(csa, x2, pos, m, k)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


@pytest.mark.parametrize("B,T,cap,k,pos", [
    (1, 64, 70000, 2048, [279900]),     # prefill chunk rows held whole in registers
    (1, 16, 90000, 2048, [359900]),     # prefill chunk rows past the register chunk
    (4, 1, 32768, 1024, [131071] * 4),  # decode rows
])
def test_fused_equals_unfused_on_inexact_scores(csa, B, T, cap, k, pos):
    """Non-dyadic head weights and wide block scales make the scores inexact in fp32;
    the fused call must still select exactly what csa_topk selects on the scores
    csa_indexer_scores writes."""
    say(f"indexer_topk vs unfused (inexact) B={B} T={T} cap={cap} k={k}")
    H_I, d_I, m = 8, 128, 4
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=cap + T)
    (r,) = streams(123, cap, 1)
    x["w"] = r.uniform(0.1, 3.0, size=x["w"].shape).astype(np.float32)
    x["q_e8m0"] = r.integers(110, 140, size=x["q_e8m0"].shape).astype(np.uint8)
    x["k_e8m0"] = r.integers(110, 140, size=x["k_e8m0"].shape).astype(np.uint8)
    pos = np.array(pos, np.int32)
    d = _dev(x)
    scores = csa.csa_indexer_scores(*d, t_i32(pos), m)
    ref = h(csa.csa_topk(scores, t_i32(pos), m, k))
    got = h(csa.csa_indexer_topk(*d, t_i32(pos), m, k))
    torch.cuda.synchronize()
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]


@pytest.mark.parametrize("cap,cluster,k", [
    (60000, 600, 500),     # the cluster overflows its (block, row) candidate staging: fallback path
    (200000, 100, 60),     # the cluster fits the staging: the selection resolves the tie class
])
def test_fused_clustered_candidates(csa, cap, cluster, k):
    """Chunk rows on the threshold path whose best entries sit together: rows 0 and 1
    have an all-ones query (w = 1), so a run of `cluster` consecutive keys with every
    element 24 scores the maximum, all tied, and the rest score by their random keys.  With
    600 such entries one block of the candidate pass finds more than its staging
    holds and the row must take the full fallback; with 100 they fit and the
    selection orders the tie class by entry.  Row 2 has a random query."""
    say(f"indexer_topk clustered candidates cap={cap} cluster={cluster} k={k}")
    B, T, H_I, d_I, m = 1, 3, 4, 64, 4
    x = indexer_inputs(B, T, cap, H_I, d_I, seed=cap + cluster)
    x["q_codes"][0, :2] = 0x22                               # rows 0, 1: every element +1
    x["q_e8m0"][0, :2] = 127
    x["w"][0, :2] = 1.0
    kc = x["k_codes"].copy()
    ke = x["k_e8m0"].copy()
    c0 = 20100
    kc[0, c0:c0 + cluster] = 0x77                            # the cluster: every element 6 * 2^2,
    ke[0, c0:c0 + cluster] = 129                             # above any random key's sum
    x2 = dict(x, k_codes=kc, k_e8m0=ke)
    pos = np.array([4 * cap - 4], np.int32)
    s = indexer_scores(x2["q_codes"], x2["q_e8m0"], x2["w"], kc, ke, pos, m)
    ref = topk(s.astype(np.float32), pos, m, k)
    assert np.array_equal(ref[0, 0], np.arange(c0, c0 + k))   # the lowest-index k of the tied cluster
    got = _fused(csa, x2, pos, m, k)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
