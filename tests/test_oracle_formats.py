"""Pins of the oracle's number formats against library routines and the format definitions."""
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle.formats import (bf16_decode, bf16_encode, bf16_round, e2m1_decode, e4m3_decode,
                            e4m3_encode, e4m3_round, mxfp4_decode, unpack_nibbles)

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
