"""Pins of the oracle's QSA indexer (pooled index keys, scores, selection of a budget of positions).

Against the offload page: the pooled key size (1 x (128/4) x 2 bytes = 64 bytes; with the 2-byte slot, 66 bytes
per token per layer; ``tests/golden/p2_index_bytes.csv``). Against the mathematics: the pooled value is the bf16
rounding of the exact mean (worked out with rationals), a score is the exact dot product where every partial
sum is representable, within the recursive-summation bound of the exact (fsum) value otherwise, and follows
channel order where the order matters; the chosen set equals a brute-force rank count on tiny inputs with many
ties, for every budget and count of forced recent positions.
"""
import csv
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import indexer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLD, "p2_index_bytes.csv")) as f:
        return {r["quantity"]: int(r["value"]) for r in csv.DictReader(l for l in f if not l.startswith("#"))}


def bf16(x):
    """float -> bf16 bits by round to nearest even, through fp32 (numpy's fp32 conversion is RNE)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rne_bf16_of_fraction(fr: Fraction) -> int:
    """bf16 bits of the rational fr by round to nearest even, worked out exactly (normal range only)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 7)          # in [128, 256): 8 significant bits
    m = math.floor(scaled)
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    if m == 256:
        m, e = 128, e + 1
    return sign | ((e + 127) << 7) | (m - 128)


def test_index_bytes_match_the_page():
    g = _golden()
    assert g["indexer_head_dim"] // g["indexer_compress_ratio"] == indexer.POOLED
    assert indexer.index_token_bytes(g["indexer_head_dim"], g["indexer_compress_ratio"]) == g["pooled_key_bytes"]
    assert indexer.KEY_BYTES == g["pooled_key_bytes"]
    assert g["pooled_key_bytes"] + g["slot_bytes"] == g["resident_bytes_per_token_per_layer"]
    assert oracle.sizes.bf16_token_bytes(2, 256) == g["full_row_bytes"]
    # the cache's index region: 64 bytes per position
    cfg = dict(n_layers=1, max_seqs=1, capacity=1000, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=8, v_bits=8,
               kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, index_dim=128, index_pool=4)
    lay = oracle.layout.slab_layout(cfg)
    assert lay["index"][1] == 1024 * g["pooled_key_bytes"]
    no_index = dict(cfg, index_dim=0)
    assert oracle.layout.slab_layout(no_index)["index"][1] == 0


def test_pooling_is_the_rounded_exact_mean():
    rng = np.random.default_rng(0)
    for ratio in (1, 2, 4, 8):
        # values k/16 with |k| <= 255 are bf16 values (8 significant bits) and every fp32 partial sum of up to 8
        # of them is exact, so the mean is exact before rounding
        raw = rng.integers(-255, 256, size=(40, 32 * ratio)) / 16.0
        bits = bf16(raw)
        assert np.array_equal(f32(bits), raw.astype(np.float32))       # inputs are bf16 values
        got = indexer.pool_keys(bits, ratio)
        for n in range(40):
            for i in range(32):
                fr = sum(Fraction(float(x)) for x in f32(bits[n, i * ratio:(i + 1) * ratio])) / ratio
                assert int(got[n, i]) == rne_bf16_of_fraction(fr), (ratio, n, i)


def test_pooling_ties_round_to_even_and_constants_stay():
    # mean 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0; 1 + 3 * 2^-8 -> 1 + 2^-6
    row = np.array([[1.0, 1.0, 1.0, 1.0 + 4 * 2 ** -8] + [1.0 + 3 * 2 ** -8] * 4 + [2.5] * 120], dtype=np.float64)
    bits = np.concatenate([bf16(row[:, :4]), bf16(np.full((1, 4), 1.0)), bf16(row[:, 8:])], axis=1)
    bits[0, 4:8] = [0x3F80, 0x3F80, 0x3F80 + 1, 0x3F80 + 2]     # mean 1 + 3 * 2^-9 * 4 / 4 ... exact below
    got = indexer.pool_keys(bits, 4)
    fr0 = sum(Fraction(float(x)) for x in f32(bits[0, :4])) / 4
    assert fr0 == 1 + Fraction(1, 256)
    assert int(got[0, 0]) == 0x3F80                               # halfway -> even mantissa (1.0)
    fr1 = sum(Fraction(float(x)) for x in f32(bits[0, 4:8])) / 4
    assert int(got[0, 1]) == rne_bf16_of_fraction(fr1)
    assert all(int(got[0, i]) == int(bf16(np.float32(2.5))) for i in range(2, 32))


def test_scores_exact_on_small_integers():
    rng = np.random.default_rng(1)
    q = rng.integers(-20, 21, size=32).astype(np.float64)
    k = rng.integers(-20, 21, size=(200, 32)).astype(np.float64)
    s = indexer.scores(bf16(q), bf16(k))
    assert np.array_equal(s.astype(np.float64), k @ q)


def test_scores_within_the_summation_bound():
    rng = np.random.default_rng(2)
    q = bf16(rng.standard_normal(32))
    k = bf16(rng.standard_normal((500, 32)) * np.exp(rng.uniform(-6, 6, size=(1, 32))))
    s = indexer.scores(q, k).astype(np.float64)
    qf, kf = f32(q).astype(np.float64), f32(k).astype(np.float64)
    u = 2.0 ** -24
    gamma = 31 * u / (1 - 31 * u)
    for t in range(500):
        prods = [qf[i] * kf[t, i] for i in range(32)]
        exact = math.fsum(prods)
        assert abs(s[t] - exact) <= gamma * math.fsum(abs(p) for p in prods) + 1e-300


def test_scores_follow_channel_order():
    # products 2^24, 1, -2^24, 1, 0...: in channel order (2^24 + 1) rounds to 2^24, then 0, then 1; exact sum is 2
    q = np.zeros(32)
    q[:4] = 1.0
    k = np.zeros((1, 32))
    k[0, :4] = [2.0 ** 24, 1.0, -(2.0 ** 24), 1.0]
    assert float(indexer.scores(bf16(q), bf16(k))[0]) == 1.0
    k[0, :4] = [1.0, 1.0, 2.0 ** 24, -(2.0 ** 24)]                # same products, another order: exact 2
    assert float(indexer.scores(bf16(q), bf16(k))[0]) == 2.0


def test_zero_score_is_positive_zero():
    q = np.zeros(32)
    q[0] = 1.0
    k = np.zeros((1, 32))
    k[0, 0] = -0.0
    s = indexer.scores(bf16(q), bf16(np.array([[-(0.0)] * 32])))
    assert not np.signbit(s[0])


def _brute(score, length, budget, n_recent):
    m = max(length - n_recent, 0)
    k = budget - (length - m)
    chosen = []
    for t in range(m):
        beat = sum(1 for u in range(m) if score[u] > score[t] or (score[u] == score[t] and u < t))
        if beat < k:
            chosen.append(t)
    return sorted(chosen) + list(range(m, length))


@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_a_rank_count_on_tiny_inputs(seed):
    rng = np.random.default_rng(10 + seed)
    for length in range(0, 13):
        score = rng.integers(-2, 3, size=max(length, 1)).astype(np.float32)   # many ties
        for budget in range(1, 14):
            for n_recent in range(0, budget + 1):
                got = indexer.select(score, length, budget, n_recent)
                want = _brute(score, length, budget, n_recent)
                assert list(got[:len(want)]) == want, (length, budget, n_recent)
                assert all(x == -1 for x in got[len(want):])
                assert len(want) == min(length, budget)


def test_cache_index_select_uses_the_stored_keys():
    cfg = dict(n_layers=1, max_seqs=2, capacity=600, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=8, v_bits=8,
               kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, index_dim=128, index_pool=4)
    o = oracle.OracleCache(cfg)
    rng = np.random.default_rng(3)
    kv = bf16(rng.standard_normal((500, 2, 256)))
    raw = bf16(rng.standard_normal((500, 128)))
    o.append(0, [0, 1], [300, 200], kv, kv)
    o.index_write(0, [0, 1], [300, 200], raw)
    q = bf16(rng.standard_normal((2, 32)))
    got = o.index_select(0, [0, 1], q, 64, 16)
    for i, (lo, n) in enumerate(((0, 300), (300, 200))):
        pooled = indexer.pool_keys(raw[lo:lo + n], 4)
        sc = indexer.scores(q[i], pooled[:n - 16])
        assert np.array_equal(got[i], indexer.select(sc, n, 64, 16))
    # keys written in two chunks equal one write
    o2 = oracle.OracleCache(cfg)
    o2.append(0, [0], [100], kv[:100], kv[:100])
    o2.index_write(0, [0], [100], raw[:100])
    o2.append(0, [0], [200], kv[100:300], kv[100:300])
    o2.index_write(0, [0], [200], raw[100:300])
    assert np.array_equal(o2.st(0, 0).ikey, o.st(0, 0).ikey)
