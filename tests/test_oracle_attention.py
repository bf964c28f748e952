"""Pins of the oracle's attention: brute force, closed forms and sparse/dense relations."""
import math

import numpy as np
import pytest

from oracle import OracleCache, attend, decode_reference, sparse_reference, multi_query_reference
from workloads import small_tokens, small_query


def brute(q, k, v, scale):
    """Scalar reference with math.fsum / math.exp: q [Hq, D], k/v [T, Hkv, D] (Python floats)."""
    hq, d = q.shape
    t_len, hk, _ = k.shape
    group = hq // hk
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h // group
        s = [scale * math.fsum(float(q[h, i]) * float(k[t, g, i]) for i in range(d)) for t in range(t_len)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        den = math.fsum(w)
        for i in range(d):
            out[h, i] = math.fsum(w[t] * float(v[t, g, i]) for t in range(t_len)) / den
    return out


@pytest.mark.parametrize("hq,hk,t_len", [(4, 2, 7), (4, 4, 33), (8, 1, 64), (2, 2, 1)])
def test_attend_brute_force(hq, hk, t_len):
    rng = np.random.default_rng(hq * 100 + t_len)
    q = rng.standard_normal((hq, 32))
    k = rng.standard_normal((t_len, hk, 32)) * 2
    v = rng.standard_normal((t_len, hk, 32)) * 5
    np.testing.assert_allclose(attend(q, k, v, 0.3), brute(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    k = np.repeat(rng.standard_normal((1, 2, 32)), 10, axis=0)
    v = rng.standard_normal((10, 2, 32))
    out = attend(rng.standard_normal((4, 32)), k, v, 1.0)
    np.testing.assert_allclose(out[:2], np.repeat(v[:, 0].mean(0)[None], 2, 0), atol=1e-13)
    np.testing.assert_allclose(out[2:], np.repeat(v[:, 1].mean(0)[None], 2, 0), atol=1e-13)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    q = np.zeros((2, 32))
    q[:, 0] = 1.0
    k = rng.standard_normal((20, 1, 32)) * 0.01
    k[13, 0, 0] = 100.0                     # score gap > 60 at scale 1
    v = rng.standard_normal((20, 1, 32))
    out = attend(q, k, v, 1.0)
    np.testing.assert_allclose(out, np.repeat(v[13:14, 0], 2, 0), atol=1e-20)


def test_gqa_head_mapping():
    # query heads 0,1 read KV head 0; heads 2,3 read KV head 1
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((9, 2, 32))
    v = rng.standard_normal((9, 2, 32))
    out = attend(q, k, v, 0.5)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(out[h], attend(q[h:h + 1], k[:, g:g + 1], v[:, g:g + 1], 0.5)[0], atol=1e-14)


def _cache(tail_len=64, tail_dtype=1, n=300):
    c = dict(n_layers=1, max_seqs=1, capacity=512, n_q_heads=16, n_kv_heads=2, head_dim=256,
             k_bits=6, v_bits=5, kvarn=0, tail_len=tail_len, tail_slack=32, tail_dtype=tail_dtype)
    k, v = small_tokens(11, n, 2, 256)
    o = OracleCache(c)
    o.append(0, [0], [n], k, v)
    o.tail_evict(0, [0])
    return o, k, v, c


def test_sparse_with_all_positions_equals_dense():
    o, *_ = _cache()
    q = small_query(1, 1, 16, 256)
    dense = decode_reference(o, 0, [0], q)
    perm = np.random.default_rng(4).permutation(300)[None, :]
    sparse = sparse_reference(o, 0, [0], q, perm)
    np.testing.assert_allclose(sparse, dense, atol=1e-12, rtol=0)


def test_sparse_equals_dense_over_cache_holding_only_those_positions():
    o, k, v, c = _cache(tail_len=0)
    pos = np.sort(np.random.default_rng(5).choice(300, 40, replace=False))
    q = small_query(2, 1, 16, 256)
    sparse = sparse_reference(o, 0, [0], q, pos[None, :])
    only = OracleCache(c)
    only.append(0, [0], [40], k[pos], v[pos])
    dense = decode_reference(only, 0, [0], q)
    np.testing.assert_allclose(sparse, dense, atol=1e-12, rtol=0)
    perm = np.random.default_rng(6).permutation(pos)
    np.testing.assert_allclose(sparse_reference(o, 0, [0], q, perm[None, :]), sparse, atol=1e-12, rtol=0)


def test_default_scale_is_inverse_sqrt_dim():
    o, *_ = _cache()
    q = small_query(3, 1, 16, 256)
    np.testing.assert_array_equal(decode_reference(o, 0, [0], q, 0.0), decode_reference(o, 0, [0], q, 1 / 16))


def _mq(seed, n_seqs, n_q):
    return small_query(seed, n_seqs * n_q, 16, 256).reshape(n_seqs, n_q, 16, 256)


def test_multi_query_of_one_is_dense_decode():
    o, *_ = _cache()
    q = _mq(7, 1, 1)
    np.testing.assert_array_equal(multi_query_reference(o, 0, [0], q)[:, 0], decode_reference(o, 0, [0], q[:, 0]))


def test_multi_query_equals_dense_decode_of_each_prefix():
    """Without a ring the cached codes of a prefix do not depend on what follows: query t of T equals dense decode
    over a fresh cache that holds only the first len - T + t + 1 tokens."""
    o, k, v, c = _cache(tail_len=0)
    q = _mq(8, 1, 5)
    got = multi_query_reference(o, 0, [0], q)
    for t in range(5):
        n_t = 300 - 5 + t + 1
        prefix = OracleCache(c)
        prefix.append(0, [0], [n_t], k[:n_t], v[:n_t])
        np.testing.assert_allclose(got[0, t], decode_reference(prefix, 0, [0], q[:, t])[0], atol=1e-12, rtol=0)


def test_multi_query_masked_softmax_brute_force():
    """The causal reading as a mask over all cached positions (masked scores at -inf), summed with math.fsum, on a
    cache that mixes body rows and bf16 ring rows."""
    c = dict(n_layers=1, max_seqs=1, capacity=128, n_q_heads=4, n_kv_heads=2, head_dim=256,
             k_bits=4, v_bits=3, kvarn=0, tail_len=32, tail_slack=32, tail_dtype=1)
    k, v = small_tokens(12, 45, 2, 256)
    o = OracleCache(c)
    o.append(0, [0], [45], k, v)
    o.tail_evict(0, [0])
    n_q = 3
    q = small_query(9, n_q, 4, 256).reshape(1, n_q, 4, 256)
    got = multi_query_reference(o, 0, [0], q)
    kd, vd = o.dequantized(0, 0, np.arange(45))
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in range(n_q):
        for h in range(4):
            g = h // 2
            s = [math.fsum(float(qf[0, t, h, i]) * float(kd[j, g, i]) for i in range(256)) / 16.0
                 if j <= 45 - n_q + t else -math.inf for j in range(45)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            den = math.fsum(w)
            want = [math.fsum(w[j] * float(vd[j, g, i]) for j in range(45)) / den for i in range(256)]
            np.testing.assert_allclose(got[0, t, h], want, atol=1e-12, rtol=0)


def test_multi_query_needs_as_many_positions_as_queries():
    o, *_ = _cache(n=3)
    with pytest.raises(ValueError):
        multi_query_reference(o, 0, [0], _mq(1, 1, 4))


# ---- chunked prefill: the query of new token j attends causally to the cache as it stands after the append

def _bf16_of(x):
    from workloads import bf16_bits
    return bf16_bits(np.asarray(x, dtype=np.float32))


def test_prefill_with_zero_keys_is_the_running_mean_of_values():
    """Closed form: with all keys zero every score is equal, so the query at position p returns the mean of the
    stored V over positions 0..p. With a bf16 ring wider than the context V is stored exactly, so the mean is of
    the inputs themselves; two sequences with ragged chunks (one of them empty) check the packed row order."""
    from oracle import prefill_reference
    c = dict(n_layers=1, max_seqs=3, capacity=256, n_q_heads=4, n_kv_heads=2, head_dim=256,
             k_bits=4, v_bits=4, kvarn=0, tail_len=200, tail_slack=32, tail_dtype=1)
    o = OracleCache(c)
    rng = np.random.default_rng(5)
    vals = {0: [], 2: []}
    for n_new in ([13, 0], [7, 20], [1, 3]):
        total = sum(n_new)
        k = _bf16_of(np.zeros((total, 2, 256)))
        v = _bf16_of(rng.standard_normal((total, 2, 256)))
        q = small_query(int(total), total, 4, 256)
        o.append(0, [0, 2], n_new, k, v)
        got = prefill_reference(o, 0, [0, 2], n_new, q)
        row = 0
        for i, sid in enumerate((0, 2)):
            vf = (v[row:row + n_new[i]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            for j in range(n_new[i]):
                vals[sid].append(vf[j])
                hist = np.stack(vals[sid])                    # positions 0 .. p of this sequence
                want = hist.mean(axis=0)                      # [Hkv, D]
                for h in range(4):
                    np.testing.assert_allclose(got[row + j, h], want[h // 2], atol=1e-12, rtol=0)
            row += n_new[i]


def test_prefill_rows_equal_dense_decode_of_fresh_prefix_caches():
    """Without a ring the stored codes of a prefix do not depend on what follows: row j of a chunk equals dense
    decode over a fresh cache holding only positions 0..p (p its position), appended in the same chunks."""
    from oracle import prefill_reference
    c = dict(n_layers=1, max_seqs=1, capacity=512, n_q_heads=16, n_kv_heads=2, head_dim=256,
             k_bits=5, v_bits=3, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0)
    k, v = small_tokens(41, 140, 2, 256)
    q = small_query(42, 140, 16, 256)
    o = OracleCache(c)
    o.append(0, [0], [100], k[:100], v[:100])
    o.append(0, [0], [40], k[100:], v[100:])
    rows = [0, 17, 39]
    got = prefill_reference(o, 0, [0], [40], q[100:], rows=rows)
    for r_i, j in enumerate(rows):
        p = 100 + j
        fresh = OracleCache(c)
        fresh.append(0, [0], [100], k[:100], v[:100])
        fresh.append(0, [0], [j + 1], k[100:p + 1], v[100:p + 1])
        want = decode_reference(fresh, 0, [0], q[100 + j][None])[0]
        np.testing.assert_allclose(got[r_i], want, atol=1e-12, rtol=0)


def test_prefill_last_row_is_dense_decode_of_the_whole_cache():
    from oracle import prefill_reference
    o, *_ = _cache()
    n, _ = o.lengths(0, 0)
    q = small_query(3, 4, 16, 256)
    got = prefill_reference(o, 0, [0], [4], q, rows=[3])
    np.testing.assert_array_equal(got[0], decode_reference(o, 0, [0], q[3][None])[0])
