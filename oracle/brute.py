"""Pure-Python loop versions of every step, for tiny inputs (test infrastructure).

Written independently of the numpy modules (own format decoding from the bit
fields, own loops, Python floats = IEEE fp64) so that the two can check each
other.  Same definitions and readings as the numpy modules; see their headers
for the pages each step follows.
"""
import math
import struct


def bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e2m1(code):
    code = int(code)
    sign = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    mnt = code & 1
    if e == 0:
        return sign * 0.5 * mnt                  # subnormal: m * 2^(1-1) / 2
    return sign * math.ldexp(1.0 + 0.5 * mnt, e - 1)


def e4m3(code):
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    mnt = code & 7
    if e == 15 and mnt == 7:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(mnt / 8.0, -6)
    return sign * math.ldexp(1.0 + mnt / 8.0, e - 7)


def mxfp4_vector(packed_row, e8m0_row):
    """One MXFP4 vector -> list of floats."""
    out = []
    for i, byte in enumerate(packed_row):
        for nib in (int(byte) & 15, int(byte) >> 4):
            j = len(out)
            out.append(e2m1(nib) * math.ldexp(1.0, int(e8m0_row[j // 32]) - 127))
    return out


def compress(K, V, logits, m):
    """K, V: nested lists [B][L][d] floats; logits [B][L] -> (Khat, Vhat) [B][L//m][d]."""
    Kh, Vh = [], []
    for b in range(len(K)):
        kb, vb = [], []
        for e in range(len(K[b]) // m):
            z = [logits[b][e * m + j] for j in range(m)]
            mx = max(z)
            ex = [math.exp(x - mx) for x in z]
            tot = sum(ex)
            a = [x / tot for x in ex]
            d = len(K[b][0])
            kb.append([sum(a[j] * K[b][e * m + j][c] for j in range(m)) for c in range(d)])
            vb.append([sum(a[j] * V[b][e * m + j][c] for j in range(m)) for c in range(d)])
        Kh.append(kb)
        Vh.append(vb)
    return Kh, Vh


def indexer(Q, w, Kx, t, m):
    """One query: Q [H][dI] floats, w [H], Kx [cap][dI] -> scores [cap] (-inf if not visible)."""
    nv = (t + 1) // m
    out = []
    for e in range(len(Kx)):
        if e >= nv:
            out.append(float("-inf"))
            continue
        s = 0.0
        for h in range(len(Q)):
            dot = 0.0
            for i in range(len(Q[h])):
                dot += Q[h][i] * Kx[e][i]
            s += w[h] * (dot if dot > 0 else 0.0)
        out.append(s)
    return out


def topk(scores, t, m, k):
    """One row -> k indices ascending, -1 padded.  Repeated max-extraction."""
    nv = (t + 1) // m
    left = list(range(nv))
    chosen = []
    while left and len(chosen) < k:
        best = left[0]
        for e in left[1:]:
            if scores[e] > scores[best]:       # strict: equal scores keep the lower index
                best = e
        chosen.append(best)
        left.remove(best)
    chosen.sort()
    return chosen + [-1] * (k - len(chosen))


def attend(qh, keys, vals, sm):
    """qh [H][d]; keys, vals [n][d] -> (O [H][d], lse [H])."""
    H, d = len(qh), len(qh[0])
    if not keys:
        return [[0.0] * d for _ in range(H)], [float("-inf")] * H
    O, L = [], []
    for h in range(H):
        lg = [sm * sum(qh[h][c] * kk[c] for c in range(d)) for kk in keys]
        mx = max(lg)
        p = [math.exp(x - mx) for x in lg]
        tot = sum(p)
        O.append([sum(p[j] * vals[j][c] for j in range(len(keys))) / tot for c in range(d)])
        L.append(mx + math.log(tot))
    return O, L


def window(t, W):
    return list(range(max(0, t - W + 1), t + 1))


def csa_attend(qh, cK, cV, sel, Kw, Vw, raw_pos0, t, W, sm):
    keys = [cK[e] for e in sel if e >= 0] + [Kw[p - raw_pos0] for p in window(t, W)]
    vals = [cV[e] for e in sel if e >= 0] + [Vw[p - raw_pos0] for p in window(t, W)]
    return attend(qh, keys, vals, sm)


def hca_attend(qh, cK, cV, m_prime, Kw, Vw, raw_pos0, t, W, sm):
    nv = (t + 1) // m_prime
    keys = [cK[e] for e in range(nv)] + [Kw[p - raw_pos0] for p in window(t, W)]
    vals = [cV[e] for e in range(nv)] + [Vw[p - raw_pos0] for p in window(t, W)]
    return attend(qh, keys, vals, sm)
