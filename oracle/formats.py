"""Number formats of the path, decoded and encoded in fp64 (test infrastructure).

Pages: the KV cache is kept in a BF16 / FP8 mix ("DeepSeek-V4 技术分析报告",
§3 核心技术拆解, 工程层); FP4 in its MXFP4 form is used on the indexer's
query-key path ("DeepSeek V4技术揭秘", §一 基础设施); FP8 here is E4M3 and FP4 is
E2M1, and FP4 -> FP8 is lossless because E4M3 has two more exponent bits
(sz-guanghua.com.cn ifanr repost "定了，DeepSeek V4首發華為芯片", the weight-precision
paragraph).  Bit-level definitions that the pages leave open follow the public
OCP specifications: OCP 8-bit FP (E4M3FN: bias 7, no infinities, S.1111.111 is
NaN, max 448) and OCP Microscaling v1.0 (E2M1 elements, 32-element blocks, one
E8M0 power-of-two scale per block, 0xFF = NaN).  Packing of two E2M1 codes per
byte is a project choice: element 2i sits in the low nibble of byte i.

Everything here is exact in fp64 (every value of these formats is a dyadic
rational with a short significand).
"""
import numpy as np

# ---------------------------------------------------------------- bf16 ------


def bf16_decode(bits):
    """uint16 bf16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _round_to_significand(x, sig_bits, min_exp):
    """Round fp64 x to the nearest value with `sig_bits` significant bits, ties to even.

    `min_exp` is the exponent of the smallest normal number of the target
    format; below it the quantum stays fixed (gradual underflow).  Works on the
    exact fp64 value, so the result is a single correctly rounded step.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, ex = np.frexp(x[nz])            # |x| = f * 2**ex, 0.5 <= f < 1
    lead = ex.astype(np.int64) - 1     # exponent of the leading bit
    lead = np.maximum(lead, min_exp)
    q = np.ldexp(1.0, lead - (sig_bits - 1))
    out[nz] = np.rint(x[nz] / q) * q   # x / q is exact (power-of-two scaling)
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    # keep the sign of zero results (e.g. -tiny rounds to -0)
    out = np.copysign(out, x)
    return out


def bf16_round(x):
    """fp64 -> nearest bf16 value (RNE), returned as float64."""
    return _round_to_significand(x, 8, -126)


def bf16_encode(x):
    """fp64 -> bf16 bit patterns (uint16), round to nearest even, one rounding."""
    y = bf16_round(x)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > 3.3895313892515355e38):
        raise ValueError("bf16 overflow")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f32_round(x):
    """fp64 -> nearest fp32 value (IEEE RNE via numpy's correctly rounded cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)

# ------------------------------------------------------------ E4M3FN -------

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 OCP E4M3FN codes -> float64.  NaN codes (0x7F, 0xFF) decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mnt = c & 0x7
    normal = s * np.ldexp(1.0 + mnt / 8.0, e - 7)
    sub = s * np.ldexp(mnt / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (mnt == 7), np.nan, v)


_E4M3_TABLE = None


def _e4m3_value_to_code():
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        vals = e4m3_decode(np.arange(256, dtype=np.uint8))
        tab = {}
        for code in range(256):
            v = vals[code]
            if np.isnan(v):
                continue
            key = (float(v), bool(np.signbit(v)))
            tab[key] = code
        _E4M3_TABLE = tab
    return _E4M3_TABLE


def e4m3_round(x):
    """fp64 -> nearest E4M3FN value (RNE), saturated to +-448; float64 out."""
    y = _round_to_significand(x, 4, -6)
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x):
    """fp64 -> E4M3FN codes (uint8), RNE with saturation at +-448."""
    y = e4m3_round(x)
    tab = _e4m3_value_to_code()
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        out[i] = tab[(float(v), bool(np.signbit(v)))]
    return out.reshape(y.shape)

# ------------------------------------------------------- E2M1 / MXFP4 ------

# OCP MX v1.0 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def e2m1_decode(nibbles):
    """4-bit E2M1 codes (0..15, bit 3 = sign) -> float64."""
    n = np.asarray(nibbles).astype(np.int64)
    mag = E2M1_MAGNITUDES[n & 0x7]
    return np.where(n & 0x8, -mag, mag)


def e8m0_decode(e):
    """E8M0 scale bytes -> 2**(e-127).  0xFF is NaN and rejected."""
    e = np.asarray(e).astype(np.int64)
    if np.any(e == 255):
        raise ValueError("E8M0 NaN scale")
    return np.ldexp(1.0, e - 127)


def unpack_nibbles(packed):
    """[..., n/2] uint8 -> [..., n] codes; element 2i = low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0x0F
    hi = p >> 4
    return np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * 2,))


def mxfp4_decode(packed, e8m0):
    """MXFP4 tensor -> float64.

    packed: [..., d/2] uint8 (two E2M1 codes per byte), e8m0: [..., d/32] uint8.
    Element i is e2m1(code_i) * 2**(e8m0[i // 32] - 127).
    """
    vals = e2m1_decode(unpack_nibbles(packed))
    d = vals.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("MXFP4 length must be a multiple of 32")
    sc = e8m0_decode(e8m0)
    if sc.shape[-1] != d // MX_BLOCK:
        raise ValueError("one scale per 32-element block")
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def mxfp4_encode(x):
    """Real values -> MXFP4 (packed E2M1 codes [..., d/2] uint8, E8M0 scales [..., d/32] uint8).

    OCP Microscaling v1.0 conversion, restated: for each 32-element block the
    shared exponent is X = floor(log2(amax)) - 2 (2 being E2M1's largest
    exponent), clamped to the E8M0 range [-127, 127]; an all-zero block takes
    X = -127 (this library's reading: the spec leaves a zero block's scale
    free).  Each element x / 2**X is rounded to the nearest E2M1 magnitude,
    a tie going to the magnitude whose mantissa bit is 0, and magnitudes past
    6 saturate to 6; the sign bit of x is kept (so -0 encodes as 0x8).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("MXFP4 length must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                       # amax = f * 2**e, f in [0.5, 1): floor(log2) = e - 1
    X = np.where(amax > 0, e - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    v = np.ldexp(blocks, -X[..., None])         # exact: a power-of-two scaling
    mag = np.abs(v)
    # nearest magnitude; among equally near ones the even code (mantissa bit 0)
    dist = np.abs(mag[..., None] - E2M1_MAGNITUDES)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    even = cand & ((np.arange(8) & 1) == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    code = np.where(mag > 6.0, 7, code)
    sign = np.signbit(v).astype(np.int64) << 3
    nib = (code | sign).reshape(x.shape).astype(np.uint8)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)
