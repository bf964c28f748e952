"""qN_0 and qN_1 block quantizers and KVarN normalization (oracle; test infrastructure only).

Block quantizer (BeeLlama.cpp v0.4.1 page, list of standard KV cache types
q2_0 .. q8_0; KVarN benchmark page, cache-size column): a block is 32
consecutive values along head_dim, stored as N-bit symmetric codes and one fp16
scale; the "_0" types carry no offset. The sizes on both pages admit exactly one
fp16 per 32 values (q8_0 = 34 bytes per 32 values = 53.1 % of bf16).

Readings (the pages give no formula): the scale is d = amax / qmax with
qmax = 2^(N-1) - 1, computed in IEEE fp32 and rounded to fp16 (round to nearest
even, saturating at 65504); codes are rne(x / d16) against the *stored* fp16
scale, clamped to [-qmax, qmax]; a block whose fp16 scale is 0 stores all-zero
codes. The stored code is the biased value u = c + 2^(N-1).

qN_1 blocks (BeeLlama.cpp v0.4.1 page, added types q2_1, q3_1, q6_1 beside q5_1; KVarN
benchmark page, cache-size column: q5_1 = 37.5 % and q8_0-q5_1 = 45.3 % of bf16, i.e.
N bits per value plus two fp16 numbers per 32 values): a scale and a minimum. Reading
(the pages give no formula): mn, mx are the block's smallest and largest value;
d = (mx - mn) / (2^N - 1) in IEEE fp32, saturating at 65504, rounded to fp16 (nearest
even); the stored minimum m16 is mn rounded to fp16 (nearest even, saturating at
+/-65504); codes u = rne((x - m16) / d16), the subtraction and the division in IEEE
fp32, clamped to [0, 2^N - 1]; a block whose fp16 scale is 0 stores all-zero codes.
The value of a code is d16 * u + m16.

KVarN (BeeLlama.cpp v0.4.1 page: "variance-normalized KV-cache quantization";
KVarN benchmark page, TL;DR): before block quantization each channel is divided
by a per-channel scale. Reading: sigma_c is the uncentered root mean square of
channel c over the first chunk appended to a (sequence, layer), computed in fp64
and rounded to fp16; 0 or non-finite gives 1; the result is clamped to
[2^-14, 65504]. Normalized values are f32(x / f32(sigma16)).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
QMAX = {n: (1 << (n - 1)) - 1 for n in range(2, 9)}
F16_MAX = np.float32(65504.0)


def f16_rne(x) -> np.ndarray:
    """fp32 (or fp64) -> fp16 with round-to-nearest-even (numpy's conversion is IEEE RNE)."""
    return np.asarray(x).astype(np.float16)


def quantize_blocks(x: np.ndarray, n_bits: int):
    """Quantize fp32 values along the last axis in blocks of 32.

    x: float32 [..., D] with D % 32 == 0.
    Returns (u, d16): u uint8 [..., D] biased codes c + 2^(N-1); d16 float16 [..., D/32].
    """
    assert 2 <= n_bits <= 8
    x = np.asarray(x, dtype=np.float32)
    d_total = x.shape[-1]
    assert d_total % BLOCK == 0
    xb = x.reshape(*x.shape[:-1], d_total // BLOCK, BLOCK)
    qmax = np.float32(QMAX[n_bits])
    amax = np.max(np.abs(xb), axis=-1)                       # exact in fp32
    d = amax / qmax                                           # IEEE fp32 division
    d = np.minimum(d, F16_MAX)                                # saturate before rounding
    d16 = f16_rne(d)                                          # RNE to fp16
    d32 = d16.astype(np.float32)                              # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        q = xb / d32[..., None]                               # IEEE fp32 division
    c = np.rint(q)                                            # round half to even
    c = np.clip(c, -qmax, qmax)
    c = np.where((d16 == 0)[..., None], np.float32(0), c)    # zero scale -> zero codes
    u = (c.astype(np.int32) + (1 << (n_bits - 1))).astype(np.uint8)
    # a zero scale is stored as +0
    d16 = np.where(d16 == 0, np.float16(0), d16)
    return u.reshape(x.shape), d16


def quantize_blocks_min(x: np.ndarray, n_bits: int):
    """qN_1: quantize fp32 values along the last axis in blocks of 32 with a scale and a minimum.

    x: float32 [..., D] with D % 32 == 0.
    Returns (u, d16, m16): u uint8 [..., D] codes in [0, 2^N - 1]; d16, m16 float16 [..., D/32].
    """
    assert 2 <= n_bits <= 8
    x = np.asarray(x, dtype=np.float32)
    d_total = x.shape[-1]
    assert d_total % BLOCK == 0
    xb = x.reshape(*x.shape[:-1], d_total // BLOCK, BLOCK)
    levels = np.float32((1 << n_bits) - 1)
    mn = np.min(xb, axis=-1)                                   # exact
    mx = np.max(xb, axis=-1)
    d = (mx - mn) / levels                                     # IEEE fp32 subtraction and division
    d = np.minimum(d, F16_MAX)
    d16 = f16_rne(d)
    m16 = f16_rne(np.clip(mn, -F16_MAX, F16_MAX))
    d32 = d16.astype(np.float32)
    m32 = m16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb - m32[..., None]) / d32[..., None]             # IEEE fp32 subtraction, then division
    c = np.clip(np.rint(q), np.float32(0), levels)
    c = np.where((d16 == 0)[..., None], np.float32(0), c)
    d16 = np.where(d16 == 0, np.float16(0), d16)
    return c.astype(np.uint8).reshape(x.shape), d16, m16


def dequantize_blocks_min(u: np.ndarray, d16: np.ndarray, m16: np.ndarray) -> np.ndarray:
    """fp64 values d16 * u + m16 for qN_1 codes [..., D], scales and minima [..., D/32]."""
    d = np.repeat(np.asarray(d16, dtype=np.float64), BLOCK, axis=-1)
    m = np.repeat(np.asarray(m16, dtype=np.float64), BLOCK, axis=-1)
    return np.asarray(u, dtype=np.float64) * d + m


def dequantize_blocks(u: np.ndarray, d16: np.ndarray, n_bits: int) -> np.ndarray:
    """Exact fp64 values (u - 2^(N-1)) * d16 for codes [..., D] and scales [..., D/32]."""
    c = np.asarray(u, dtype=np.int64) - (1 << (n_bits - 1))
    d = np.repeat(np.asarray(d16, dtype=np.float64), BLOCK, axis=-1)
    return c.astype(np.float64) * d


def kvarn_sigma(x_f32: np.ndarray) -> np.ndarray:
    """Per-channel fp16 normalization scale from a chunk of tokens.

    x_f32: float32 [n, ..., D] (the first chunk appended); returns float16 [..., D].
    sigma_c = sqrt(mean_t x_tc^2) in fp64, RNE to fp16; 0 / non-finite -> 1;
    clamped to [2^-14, 65504].
    """
    x = np.asarray(x_f32, dtype=np.float64)
    n = x.shape[0]
    ms = np.sum(x * x, axis=0) / float(n)                    # every x^2 is exact in fp64
    s = np.sqrt(ms)
    bad = (s == 0) | ~np.isfinite(s)
    s16 = f16_rne(np.where(bad, 1.0, s))
    s16 = s16.astype(np.float32)
    s16 = np.clip(s16, np.float32(2.0 ** -14), F16_MAX)
    return s16.astype(np.float16)


def normalize(x_f32: np.ndarray, sigma16: np.ndarray) -> np.ndarray:
    """y = f32(x / f32(sigma16)) channel-wise (IEEE fp32 division)."""
    return (np.asarray(x_f32, dtype=np.float32) / sigma16.astype(np.float32)).astype(np.float32)
