"""Pins of the oracle's number formats against library routines and the format definitions."""
import os

import numpy as np
import pytest
import torch

from oracle import brute
from csa_synth import mxfp4_random, streams
from oracle.formats import (bf16_decode, bf16_encode, bf16_round, e2m1_decode, e4m3_decode,
                            e4m3_encode, e4m3_round, mxfp4_decode, mxfp4_encode, unpack_nibbles)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name), encoding="utf-8"):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin]))
    assert np.nanmax(got) == 448.0


def test_e4m3_encode_matches_torch_rne():
    r = np.random.default_rng(7)
    x = np.concatenate([r.standard_normal(20000) * 40,
                        r.uniform(-448, 448, 5000),
                        r.standard_normal(5000) * 1e-2]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_round(x.astype(np.float64))
    assert np.array_equal(ref, got)
    codes = e4m3_encode(x[:2000].astype(np.float64))
    assert np.array_equal(e4m3_decode(codes), got[:2000])


def test_e4m3_saturates():
    assert e4m3_round(np.array([460.0, 1e6, -500.0])).tolist() == [448.0, 448.0, -448.0]


def test_bf16_encode_matches_torch_on_fp32():
    r = np.random.default_rng(8)
    x = (r.standard_normal(50000) * np.exp2(r.integers(-30, 30, 50000))).astype(np.float32)
    # exact ties: low 16 bits 0x8000
    t = (r.integers(0, 2**31, 2000, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    t &= np.uint32(0x7F7FFFFF)
    x = np.concatenate([x, t.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_encode(x.astype(np.float64))
    assert np.array_equal(ref, got)
    assert np.array_equal(bf16_decode(got), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def test_bf16_round_single_rounding_from_fp64():
    # 1 + 2^-8 is exactly half-way between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1.
    # 1 + 2^-8 + 2^-40 lies just above the tie: must round up.  Rounding fp64 -> fp32 -> bf16
    # would lose the 2^-40 and round down (double rounding).
    x = np.array([1 + 2.0**-8, 1 + 2.0**-8 + 2.0**-40, 1 + 3 * 2.0**-8, -(1 + 2.0**-8)])
    assert bf16_round(x).tolist() == [1.0, 1 + 2.0**-7, 1 + 4 * 2.0**-8, -1.0]


def test_e2m1_table_matches_bit_field_definition():
    # OCP MX E2M1: sign | 2 exponent bits (bias 1) | 1 mantissa bit; exponent 0 is subnormal.
    for code in range(16):
        s = -1.0 if code & 8 else 1.0
        e, mnt = (code >> 1) & 3, code & 1
        v = s * (mnt * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + mnt / 2))
        assert e2m1_decode(np.array([code]))[0] == v
        assert brute.e2m1(code) == v


def test_page_format_facts():
    g = _golden("formats.txt")
    # exponent / mantissa widths as visible in the decoded value sets
    e4 = e4m3_decode(np.arange(256, dtype=np.uint8))
    e4 = e4[np.isfinite(e4) & (e4 > 0)]
    binades4 = np.unique(np.floor(np.log2(e4)))
    normal4 = e4[e4 >= 2.0**-6]
    assert len(np.unique(normal4[(normal4 >= 1) & (normal4 < 2)])) == 2 ** g["fp8_mantissa_bits"]
    e2 = e2m1_decode(np.arange(8))
    e2 = e2[e2 > 0]
    binades2 = np.unique(np.floor(np.log2(e2)))
    # 2^E - 1 normal binades + 1 subnormal binade spread (E4M3FN: 15 normal binades + 3 sub)
    assert len(binades4) == 2 ** g["fp8_exponent_bits"] - 1 + g["fp8_mantissa_bits"]
    assert len(binades2) == 2 ** g["fp4_exponent_bits"] - 1 + g["fp4_mantissa_bits"]
    assert g["fp8_exponent_bits"] - g["fp4_exponent_bits"] == g["exponent_bits_difference"]


def test_e2m1_subset_of_e4m3_and_bf16_lossless():
    """FP4 -> FP8 (and -> bf16) is lossless, as the pages state; also with MX block scales."""
    assert _golden("formats.txt")["fp4_to_fp8_lossless"] == 1
    vals = e2m1_decode(np.arange(16))
    for e in range(-6, 3):               # E4M3 normal range keeps the scaled grid exact
        x = vals * 2.0 ** e
        assert np.array_equal(e4m3_round(x), x)
        assert np.array_equal(bf16_round(x), x)
    for e in range(-126, 120, 7):        # bf16 has the exponent range of fp32
        x = vals * 2.0 ** e
        assert np.array_equal(bf16_round(x), x)


def test_mxfp4_packing_and_block_scales():
    # element 2i = low nibble, 2i+1 = high nibble; block j of 32 uses scale j
    codes = np.array([(2 * i) % 16 | (((2 * i + 1) % 16) << 4) for i in range(32)], np.uint8)
    e8 = np.array([127, 129], np.uint8)
    v = mxfp4_decode(codes, e8)
    nib = unpack_nibbles(codes)
    assert nib[:4].tolist() == [0, 1, 2, 3]
    ref = np.array([brute.e2m1(c) for c in nib], float)
    ref[32:] *= 4.0
    assert np.array_equal(v, ref)
    assert np.array_equal(v, np.array(brute.mxfp4_vector(codes, e8)))
    with pytest.raises(ValueError):
        mxfp4_decode(codes, np.array([255, 127], np.uint8))


# ---------------------------------------------------------- MXFP4 encoder ----
# OCP Microscaling v1.0 conversion: X = floor(log2(amax)) - 2, elements rounded
# to nearest E2M1 (ties to the even mantissa bit), saturated at 6.

def test_mxfp4_encode_hand_example():
    """amax 6 gives X = 0 (E8M0 127); every tie of the E2M1 grid resolved by hand:
    0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4 (even
    mantissa bit), 5.5 -> 6 (nearer), -0 keeps its sign bit."""
    x = np.zeros((1, 32))
    x[0, :12] = [6.0, -3.0, 0.75, 0.25, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, -0.0, 0.1]
    packed, e8 = mxfp4_encode(x)
    assert e8.tolist() == [[127]]
    want = [0xD7, 0x02, 0x42, 0x64, 0x76, 0x08] + [0] * 10   # codes 7,D 2,0 2,4 4,6 6,7 8,0
    assert packed[0].tolist() == want


@pytest.mark.parametrize("amax,code", [
    (1.0, 125), (6.0, 127), (7.9, 127), (8.0, 128), (2.0 ** -10, 115), (2.0 ** 100, 225),
    (0.0, 0), (2.0 ** -140, 0), (3.0 * 2.0 ** 200, 254)])
def test_mxfp4_encode_scale_rule(amax, code):
    x = np.zeros(32)
    x[5] = -amax
    packed, e8 = mxfp4_encode(x)
    assert int(e8[0]) == code
    v = mxfp4_decode(packed, e8)
    if amax == 2.0 ** -140:
        assert v[5] == 0.0                         # below the smallest scale's grid: rounds to zero
    elif amax == 3.0 * 2.0 ** 200:
        assert v[5] == -6.0 * 2.0 ** 127           # past the largest scale: saturated
    else:
        assert v[5] == -amax or (amax == 7.9 and v[5] == -6.0)


def test_mxfp4_encode_round_trips_every_representable_block():
    """Decoding, encoding and decoding again gives the same values, for blocks of
    every code mix (full range, small magnitudes only, zeros) and many scales."""
    rc, re = streams(71, 0, 2)
    for codes in (None, [0, 1, 2, 3, 8, 9, 10, 11], [0, 1, 9], [0, 8]):
        packed, e8 = mxfp4_random(rc, re, (64,), 128, codes=codes, exps=tuple(range(100, 160)))
        v = mxfp4_decode(packed, e8)
        p2, e2 = mxfp4_encode(v)
        assert np.array_equal(mxfp4_decode(p2, e2), v)


def test_mxfp4_encode_error_bound_and_monotone():
    """Each element lands within half an E2M1 step of x (steps 0.5, 1, 2 times the
    scale below 2, 4, 6) or saturates at 6; within a block the encoding is monotone."""
    (r,) = streams(72, 0, 1)
    x = r.standard_normal((200, 64)) * np.exp2(r.integers(-20, 20, (200, 1)))
    packed, e8 = mxfp4_encode(x)
    q = mxfp4_decode(packed, e8)
    sc = np.repeat(np.exp2(e8.astype(np.int64) - 127.0), 32, axis=-1)
    v = np.abs(x) / sc
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    err = np.abs(q - x) / sc
    assert np.all((err <= step / 2) | ((v > 6) & (np.abs(q) / sc == 6.0)))
    for row in range(0, 200, 17):
        for b in range(2):
            xb, qb = x[row, 32 * b:32 * b + 32], q[row, 32 * b:32 * b + 32]
            o = np.argsort(xb, kind="stable")
            assert np.all(np.diff(qb[o]) >= 0)
