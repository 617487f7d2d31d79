"""Test-side helpers: host arrays -> device tensors, and the parity tolerances.

Tolerances (derived from the arithmetic; the attention bounds are the ones the
project targets):
  * indexer scores, top-k indices: exact (value equality; -0 == +0);
  * attention outputs: max-abs 2e-2 with bf16 I/O and fp32 accumulation,
    1e-5 with fp32 I/O, each on top of half a unit in the last place of the
    output format at |O| (the rounding of the stored output itself, which no
    kernel can avoid: outputs of heavy-tailed inputs reach magnitudes where a
    bf16 half-unit alone exceeds 2e-2);
  * compressed entries: the GPU pools in fp32, so its pre-rounding value x32
    differs from the exact pool x by at most eps = (m + 4) * 2^-24 * max_j |K_j|
    (m products and m additions, each within half an fp32 ulp of a partial
    result bounded by max |K_j|, plus the weight's own rounding).  After the
    storage rounding the two stored values differ by at most one unit of the
    storage format at |x| (+eps): bf16 -> 2^(e-7), fp8 E4M3 -> scale*2^(e-3)
    with e the binade of |x| (of |x|/scale), fp32 -> 2^(e-23).
"""
import sys

import numpy as np
import torch


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def t_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def t_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev())


def t_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def t_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev())


def t_kv(x, dtype):
    return t_bf16(x) if dtype == "bf16" else t_f32(x)


def h_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def h(t):
    return t.cpu().numpy()


def binade(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    return np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -149)))


def compress_tolerance(x_exact, dtype, eps, scale=None):
    """Allowed |stored_gpu - stored_oracle| per element (dequantised values)."""
    ax = np.abs(x_exact) + eps
    if dtype == "bf16":
        return np.exp2(np.maximum(binade(ax), -133) - 7) + 2 * eps
    if dtype == "f32":
        return np.exp2(np.maximum(binade(ax), -149) - 23) + 2 * eps
    if dtype == "fp8":
        s = np.asarray(scale, dtype=np.float64)[..., None]
        y = ax / s
        return s * np.exp2(np.maximum(binade(y), -6) - 3) * 1.001 + 2 * eps
    raise ValueError(dtype)


def attention_tolerance(O_exact, io_dtype):
    """Allowed |out_gpu - O_exact| per element (see the module docstring)."""
    if io_dtype == "bf16":
        return 2e-2 + np.exp2(np.maximum(binade(O_exact), -133) - 8)
    return 1e-5 + np.exp2(np.maximum(binade(O_exact), -149) - 24)


def exact_equal(a, b):
    """Value equality of float arrays (-0 == +0, -inf == -inf, no NaN allowed)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert not np.isnan(a).any() and not np.isnan(b).any()
    return np.array_equal(a, b)
