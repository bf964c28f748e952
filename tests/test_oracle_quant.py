"""Pins of the oracle's qN_0 quantizer and KVarN normalization against the mathematics.

Nothing here re-calls the oracle's own formula to produce an expected value: the
expectations come from exact rational arithmetic (``fractions``), exhaustive
search over the code levels, closed forms and invariances.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant
from workloads import bf16_bits, bf16_to_f32


def _f32(x) -> float:
    return float(np.float32(x))


def _round_f32(fr: Fraction) -> float:
    """Correctly rounded fp32 of an exact rational (independent of numpy's division)."""
    f = float(fr)                          # correctly rounded to fp64
    c = np.float32(f)                      # may double-round; fix by checking neighbours
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        if best is None or err < best[0] or (err == best[0] and (np.float32(cand).view(np.uint32) & 1) == 0):
            best = (err, cand)
    return float(best[1])


def _round_f16(x: float) -> float:
    """Correctly rounded fp16 (RNE) of an fp32 value, by exhaustive neighbour search."""
    if x == 0:
        return 0.0
    c = np.float16(x)
    best = None
    for cand in (np.nextafter(c, np.float16(-np.inf)), c, np.nextafter(c, np.float16(np.inf))):
        if not np.isfinite(cand):
            continue
        err = abs(Fraction(float(cand)) - Fraction(x))
        if best is None or err < best[0] or (err == best[0] and (np.float16(cand).view(np.uint16) & 1) == 0):
            best = (err, cand)
    return float(best[1])


def _blocks(seed, n, scale=1.0, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32) * np.float32(scale)
    if outliers:
        x[:, 3] *= 20
    return bf16_to_f32(bf16_bits(x))


@pytest.mark.parametrize("n_bits", range(2, 9))
@pytest.mark.parametrize("scale", [0.05, 1.0, 37.0])
def test_round_trip_within_half_scale(n_bits, scale):
    x = _blocks(n_bits * 7 + int(scale * 10), 400, scale, outliers=(n_bits % 2 == 0))
    u, d16 = quant.quantize_blocks(x, n_bits)
    c = u.astype(np.int64) - (1 << (n_bits - 1))
    d = d16.astype(np.float64)[:, 0]                              # one block per row
    assert np.all(d >= 2.0 ** -14) and np.all(d < 65504)        # normal, unsaturated scales
    err = np.abs(x.astype(np.float64) - c * d[:, None])
    # d16/2 from rounding to the nearest level; 2^-24 |x| from the fp32 division
    bound = d[:, None] / 2 + 2.0 ** -24 * np.abs(x)
    assert np.all(err <= bound)
    assert np.all(np.abs(c) <= quant.QMAX[n_bits])


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_scale_is_rne_fp16_of_correctly_rounded_fp32_quotient(n_bits):
    x = _blocks(100 + n_bits, 60, 3.0)
    u, d16 = quant.quantize_blocks(x, n_bits)
    qmax = (1 << (n_bits - 1)) - 1
    for b in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[b])
        d32 = _round_f32(Fraction(amax) / qmax)
        assert float(d16[b, 0]) == _round_f16(d32)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_codes_are_nearest_level_by_exhaustive_search(n_bits):
    x = _blocks(200 + n_bits, 40, 2.0)
    u, d16 = quant.quantize_blocks(x, n_bits)
    qmax = (1 << (n_bits - 1)) - 1
    for b in range(x.shape[0]):
        d = Fraction(float(d16[b, 0]))
        for i in range(32):
            xv = Fraction(float(x[b, i]))
            dists = [(abs(xv - c * d), c) for c in range(-qmax, qmax + 1)]
            dists.sort()
            best, c_best = dists[0]
            if dists[1][0] == best:          # an exact tie: round half to even
                c_best = dists[0][1] if dists[0][1] % 2 == 0 else dists[1][1]
            q = xv / d
            frac = q - math.floor(q)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20):
                continue                      # fp32 division may legitimately land on the tie
            assert int(u[b, i]) - (1 << (n_bits - 1)) == c_best, (b, i)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_power_of_two_grid_is_exact(n_bits):
    qmax = (1 << (n_bits - 1)) - 1
    rng = np.random.default_rng(n_bits)
    for k in (-10, -3, 0, 4, 9):
        c = rng.integers(-qmax, qmax + 1, size=(8, 32))
        c[:, 5] = qmax * np.where(rng.random(8) < 0.5, -1, 1)     # amax hits qmax
        x = (c * 2.0 ** k).astype(np.float32)
        u, d16 = quant.quantize_blocks(x, n_bits)
        assert np.all(d16.astype(np.float64) == 2.0 ** k)      # one block per row
        assert np.array_equal(u.astype(np.int64) - (1 << (n_bits - 1)), c)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_zero_block_and_sign_symmetry(n_bits):
    z = np.zeros((2, 32), dtype=np.float32)
    u, d16 = quant.quantize_blocks(z, n_bits)
    assert np.all(u == (1 << (n_bits - 1)))
    assert np.all(d16.view(np.uint16) == 0)
    x = _blocks(300 + n_bits, 50, 1.5)
    u1, d1 = quant.quantize_blocks(x, n_bits)
    u2, d2 = quant.quantize_blocks(-x, n_bits)
    off = 1 << (n_bits - 1)
    assert np.array_equal(d1.view(np.uint16), d2.view(np.uint16))
    assert np.array_equal(u1.astype(int) - off, -(u2.astype(int) - off))


def test_tiny_and_huge_scales():
    # scale below half the smallest fp16 subnormal -> zero scale, zero codes
    x = np.full((1, 32), 1e-9, dtype=np.float32)
    u, d16 = quant.quantize_blocks(x, 4)
    assert d16.view(np.uint16)[0, 0] == 0 and np.all(u == 8)
    # saturation at 65504: codes clamp to qmax
    x = np.full((1, 32), 3e38, dtype=np.float32)
    u, d16 = quant.quantize_blocks(x, 8)
    assert float(d16[0, 0]) == 65504.0 and np.all(u == 255)
    # an fp16-subnormal scale is kept (no flush) and codes stay within range
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1e-4
    x[0, 1] = -3e-5
    u, d16 = quant.quantize_blocks(x, 8)
    assert 0 < float(d16[0, 0]) < 2.0 ** -14
    assert int(u[0, 0]) - 128 == 127


def test_dequantize_exact():
    u = np.array([[0, 1, 127, 128, 255] + [128] * 27], dtype=np.uint8)
    d = np.array([0.375], dtype=np.float16)
    v = quant.dequantize_blocks(u, d, 8)
    assert list(v[0, :5]) == [-48.0, -47.625, -0.375, 0.0, 47.625]


# --------------------------------------------------------------------------- KVarN

def test_kvarn_sigma_brute_force():
    rng = np.random.default_rng(5)
    x = bf16_to_f32(bf16_bits(rng.standard_normal((37, 2, 64)).astype(np.float32) * 3))
    s = quant.kvarn_sigma(x)
    for h in range(2):
        for c in range(64):
            col = [float(v) for v in x[:, h, c]]
            ms = math.fsum(v * v for v in col) / len(col)
            ref = np.float16(math.sqrt(ms))          # fp64 -> fp16 RNE
            assert s[h, c] == ref


def test_kvarn_sigma_closed_forms():
    x = np.zeros((10, 1, 6), dtype=np.float32)
    x[:, 0, 0] = 2.5                     # constant channel: sigma = |a|
    x[:, 0, 1] = np.where(np.arange(10) % 2 == 0, 1.0, -1.0)   # +-1: sigma = 1
    x[:, 0, 2] = 0.0                     # zero channel -> 1
    x[:, 0, 3] = 1e-12                   # below fp16 range -> clamped to 2^-14
    x[:, 0, 4] = 1e6                     # above fp16 range -> 65504
    x[:, 0, 5] = -7.0
    s = quant.kvarn_sigma(x)[0].astype(np.float64)
    assert list(s) == [2.5, 1.0, 1.0, 2.0 ** -14, 65504.0, 7.0]


@pytest.mark.parametrize("n_bits", [3, 4, 6, 8])
def test_kvarn_unit_sigma_reduces_to_plain(n_bits):
    rng = np.random.default_rng(n_bits)
    x = bf16_to_f32(bf16_bits(rng.standard_normal((20, 1, 64)).astype(np.float32)))
    sig = np.ones((1, 64), dtype=np.float16)
    y = quant.normalize(x, sig)
    assert np.array_equal(y, x)
    assert np.array_equal(quant.quantize_blocks(y, n_bits)[0], quant.quantize_blocks(x, n_bits)[0])


@pytest.mark.parametrize("n_bits", [4, 5, 6])
def test_kvarn_power_of_two_channel_scaling(n_bits):
    rng = np.random.default_rng(10 + n_bits)
    x = bf16_to_f32(bf16_bits(rng.standard_normal((50, 1, 64)).astype(np.float32)))
    k = rng.integers(-4, 5, size=64)
    x2 = (x * (2.0 ** k)[None, None, :]).astype(np.float32)          # exact
    s1, s2 = quant.kvarn_sigma(x), quant.kvarn_sigma(x2)
    assert np.array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0 ** k[None, :])
    u1, d1 = quant.quantize_blocks(quant.normalize(x, s1), n_bits)
    u2, d2 = quant.quantize_blocks(quant.normalize(x2, s2), n_bits)
    assert np.array_equal(u1, u2) and np.array_equal(d1.view(np.uint16), d2.view(np.uint16))


def test_kvarn_normalized_round_trip():
    rng = np.random.default_rng(77)
    sc = np.abs(rng.standard_t(3, size=64)).astype(np.float32)
    x = bf16_to_f32(bf16_bits(rng.standard_normal((64, 1, 64)).astype(np.float32) * sc))
    s = quant.kvarn_sigma(x)
    y = quant.normalize(x, s)
    u, d16 = quant.quantize_blocks(y, 4)
    c = u.astype(np.float64) - 8
    err = np.abs(y.astype(np.float64) - c * np.repeat(d16.astype(np.float64), 32, axis=-1))
    assert np.all(err <= np.repeat(d16.astype(np.float64), 32, axis=-1) / 2 + 2.0 ** -24 * np.abs(y))


# ---- qN_1: a scale and a minimum per block (codes 0 .. 2^N - 1, value d16 * u + m16)

@pytest.mark.parametrize("n_bits", range(2, 9))
@pytest.mark.parametrize("scale", [0.05, 1.0, 37.0])
def test_qn1_round_trip_within_half_scale(n_bits, scale):
    x = _blocks(500 + n_bits * 7 + int(scale * 10), 300, scale, outliers=(n_bits % 2 == 1))
    x = x + np.float32(scale)                     # an offset the minimum absorbs
    u, d16, m16 = quant.quantize_blocks_min(x, n_bits)
    d = d16.astype(np.float64)[:, 0]
    m = m16.astype(np.float64)[:, 0]
    mn = x.astype(np.float64).min(axis=1)
    assert np.all(d >= 2.0 ** -14) and np.all(d < 65504)
    assert np.all(u <= (1 << n_bits) - 1)
    err = np.abs(x.astype(np.float64) - (u * d[:, None] + m[:, None]))
    # d16/2 to the nearest level, |m16 - mn| where the rounded minimum lies above the block's smallest value,
    # a few fp32 roundings of x - m16 and of the quotient
    bound = d[:, None] / 2 + np.abs(m - mn)[:, None] + 2.0 ** -22 * (np.abs(x) + np.abs(m)[:, None])
    assert np.all(err <= bound)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_qn1_scale_and_minimum_are_rne_fp16_of_the_exact_quantities(n_bits):
    x = _blocks(600 + n_bits, 50, 3.0) + np.float32(1.25)
    _, d16, m16 = quant.quantize_blocks_min(x, n_bits)
    levels = (1 << n_bits) - 1
    for b in range(x.shape[0]):
        mn = min(float(v) for v in x[b])
        mx = max(float(v) for v in x[b])
        diff = _round_f32(Fraction(mx) - Fraction(mn))           # the fp32 subtraction
        d32 = _round_f32(Fraction(diff) / levels)                 # then the fp32 division
        assert float(d16[b, 0]) == _round_f16(d32)
        assert float(m16[b, 0]) == _round_f16(mn)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_qn1_codes_are_nearest_level_by_exhaustive_search(n_bits):
    x = _blocks(700 + n_bits, 30, 2.0) - np.float32(0.75)
    u, d16, m16 = quant.quantize_blocks_min(x, n_bits)
    levels = (1 << n_bits) - 1
    for b in range(x.shape[0]):
        d = Fraction(float(d16[b, 0]))
        m = Fraction(float(m16[b, 0]))
        for i in range(32):
            xv = Fraction(float(x[b, i]))
            dists = sorted((abs(xv - (m + c * d)), c) for c in range(levels + 1))
            best, c_best = dists[0]
            if dists[1][0] == best:
                c_best = dists[0][1] if dists[0][1] % 2 == 0 else dists[1][1]
            q = (xv - m) / d
            frac = q - math.floor(q)
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 18):
                continue                      # fp32 arithmetic may legitimately land on either side of a tie
            assert int(u[b, i]) == c_best, (b, i)


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_qn1_power_of_two_grid_with_offset_is_exact(n_bits):
    levels = (1 << n_bits) - 1
    rng = np.random.default_rng(40 + n_bits)
    for k, off in ((-6, -3), (0, 5), (3, -2)):
        c = rng.integers(0, levels + 1, size=(6, 32))
        c[:, 0] = 0
        c[:, 7] = levels                     # the block spans the whole range
        x = ((c + off) * 2.0 ** k).astype(np.float32)
        u, d16, m16 = quant.quantize_blocks_min(x, n_bits)
        assert np.all(d16.astype(np.float64) == 2.0 ** k)
        assert np.all(m16.astype(np.float64) == off * 2.0 ** k)
        assert np.array_equal(u.astype(np.int64), c)
        assert np.array_equal(quant.dequantize_blocks_min(u, d16, m16), x.astype(np.float64))


def test_qn1_constant_block_stores_its_value_as_the_minimum():
    x = np.full((3, 32), 0.3125, dtype=np.float32)
    x[1] = -7.0
    x[2] = 0.0
    u, d16, m16 = quant.quantize_blocks_min(x, 4)
    assert np.all(u == 0)
    assert np.all(d16.view(np.uint16) == 0)
    assert list(m16[:, 0].astype(np.float64)) == [0.3125, -7.0, 0.0]


@pytest.mark.parametrize("cfg_id", [2, 3])
def test_kvarn_ordering_claims_of_the_kvarn_page(cfg_id):
    """Consistency of the KVarN reading (R4) with the KVarN benchmark page's headline ordering: KVarN 4-bit
    matches q5_0 and KVarN 6-bit matches q8_0. The page measures model KLD; with no model here the proxy is each
    channel's reconstruction error relative to its own RMS, averaged over channels, on the workloads' per-channel
    scale recipes (log-uniform and Student-t). KVarN at N bits must be no worse than qN+1_0 (4 -> q5_0) and than
    q8_0 (6 bits), and better than plain qN_0. This checks what the statistic is for; it does not pin the
    statistic itself, which the pages do not give."""
    import workloads as W
    k, v = W.kv_tokens(cfg_id, 0, 0, 0, 4096)
    for bits in (k, v):
        x = bf16_to_f32(bits)[:, 0, :]
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))

        def rel_err(xr):
            return float(np.sqrt(np.mean(np.mean((xr - x) ** 2, axis=0) / rms ** 2)))

        def plain(n):
            u, d = quant.quantize_blocks(x, n)
            return rel_err(quant.dequantize_blocks(u, d, n))

        def kvarn(n):
            sig = quant.kvarn_sigma(x)
            u, d = quant.quantize_blocks(quant.normalize(x, sig), n)
            return rel_err(quant.dequantize_blocks(u, d, n) * sig.astype(np.float64))

        k4, k6 = kvarn(4), kvarn(6)
        assert k4 <= plain(5) and k4 < plain(4), (k4, plain(4), plain(5))
        assert k6 <= plain(8) and k6 < plain(6), (k6, plain(6), plain(8))
