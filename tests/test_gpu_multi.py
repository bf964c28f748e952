"""GPU parity of multi-query decode (the last T cached positions of a sequence decoded at once, causal among
them, as when drafted tokens are verified) through the C ABI, against the oracle's fp64 result over the same
dequantized values: within 2e-3 absolute, on both layouts, every ring kind, KVarN, and queries that straddle
the body/ring boundary."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import Pair, TOL, dev, max_err
from workloads import small_tokens, small_query

pytestmark = pytest.mark.gpu


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=3, capacity=1024, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=6,
             v_bits=5, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, layout=0)
    c.update(kw)
    return c


def mq(seed, n_seqs, n_q, hq=16):
    return small_query(seed, n_seqs * n_q, hq, 256).reshape(n_seqs, n_q, hq, 256)


def run_multi(p, layer, seq_ids, q):
    got = p.gpu.decode_attn_multi(layer, seq_ids, dev(q).view(*q.shape)).cpu().numpy()
    want = oracle.multi_query_reference(p.ora, layer, seq_ids, q)
    return got, want


@pytest.mark.parametrize("layout,tail_dtype,kvarn,n_q", [
    (0, 0, 0, 1), (0, 0, 0, 8), (0, 1, 0, 5), (0, 2, 1, 8), (0, 3, 0, 2), (0, 1, 1, 8),
    (1, 0, 0, 8), (1, 1, 0, 5), (1, 2, 1, 2), (1, 3, 1, 8)])
def test_multi_query_matches_oracle(layout, tail_dtype, kvarn, n_q):
    tail = dict(tail_len=64, tail_slack=32, tail_dtype=tail_dtype) if tail_dtype else {}
    p = Pair(cfg(layout=layout, kvarn=kvarn, **tail))
    seed = 40 * layout + 10 * tail_dtype + 3 * kvarn + n_q
    k, v = small_tokens(seed, 800, 2, 256)
    p.append(1, [0, 2], [300, 170], k[:470], v[:470])
    p.evict(1, [0, 2])
    # the drafts arrive as one more chunk (ring rows when there is a ring)
    p.append(1, [0, 2], [n_q, n_q], k[470:470 + 2 * n_q], v[470:470 + 2 * n_q])
    for s in (0, 2):
        p.lengths_match(1, s)
    got, want = run_multi(p, 1, [0, 2], mq(seed, 2, n_q))
    assert max_err(got, want) <= TOL, max_err(got, want)


@pytest.mark.parametrize("tail_dtype,n_q,hq,k_bits,v_bits", [
    (0, 3, 16, 6, 5), (1, 7, 16, 2, 8), (2, 6, 8, 8, 3), (3, 3, 2, 4, 4), (1, 2, 4, 7, 2), (2, 8, 16, 3, 6)])
def test_odd_query_counts_and_group_sizes(tail_dtype, n_q, hq, k_bits, v_bits):
    """Two queries per wave without KVarN: an odd T leaves a wave with one query, and groups of 1, 2 and 4 query
    heads per KV head leave columns unused; every ring kind, several widths."""
    tail = dict(tail_len=64, tail_slack=32, tail_dtype=tail_dtype) if tail_dtype else {}
    p = Pair(cfg(n_q_heads=hq, k_bits=k_bits, v_bits=v_bits, **tail))
    seed = 90 + 7 * tail_dtype + n_q + hq
    k, v = small_tokens(seed, 900, 2, 256)
    p.append(1, [0, 1, 2], [260, 33, 401], k[:694], v[:694])
    p.evict(1, [0, 1, 2])
    p.append(1, [0, 1, 2], [n_q] * 3, k[694:694 + 3 * n_q], v[694:694 + 3 * n_q])
    got, want = run_multi(p, 1, [0, 1, 2], mq(seed, 3, n_q, hq))
    assert max_err(got, want) <= TOL, max_err(got, want)


def test_multi_query_of_one_equals_decode_attn_bit_for_bit():
    p = Pair(cfg(tail_len=64, tail_slack=32, tail_dtype=1))
    k, v = small_tokens(3, 400, 2, 256)
    p.append(0, [1], [333], k[:333], v[:333])
    p.evict(0, [1])
    q = mq(5, 1, 1)
    multi = p.gpu.decode_attn_multi(0, [1], dev(q).view(*q.shape)).cpu().numpy()
    single = p.gpu.decode_attn(0, [1], dev(q[:, 0])).cpu().numpy()
    np.testing.assert_array_equal(multi[:, 0], single)


@pytest.mark.parametrize("layout", [0, 1])
def test_queries_straddle_the_body_and_ring(layout):
    """A window of 4 and 8 queries: after an evict the first drafts sit in the body, the last in the ring."""
    p = Pair(cfg(layout=layout, tail_len=4, tail_slack=28, tail_dtype=1, k_bits=4, v_bits=4))
    k, v = small_tokens(17, 300, 2, 256)
    p.append(0, [0], [200], k[:200], v[:200])
    p.append(0, [0], [8], k[200:208], v[200:208])
    p.evict(0, [0])
    n, body = p.gpu.lengths(0, 0)
    assert n - 8 < body < n, (n, body)
    got, want = run_multi(p, 0, [0], mq(18, 1, 8))
    assert max_err(got, want) <= TOL


def test_largest_batch_of_entries_and_a_long_context():
    """8 sequences x 8 queries (64 entries in one launch, ragged lengths), then one sequence of 8k positions."""
    p = Pair(cfg(max_seqs=8, capacity=8192, n_layers=1, tail_len=32, tail_slack=32, tail_dtype=2))
    rng = np.random.default_rng(23)
    lens = [int(x) for x in rng.integers(8, 200, size=8)]
    k, v = small_tokens(24, sum(lens), 2, 256)
    p.append(0, list(range(8)), lens, k, v)
    p.evict(0, list(range(8)))
    got, want = run_multi(p, 0, list(range(8)), mq(25, 8, 8))
    assert max_err(got, want) <= TOL
    p = Pair(cfg(max_seqs=1, capacity=8192, n_layers=1, tail_len=32, tail_slack=32, tail_dtype=2))
    k, v = small_tokens(26, 8000, 2, 256)
    p.append(0, [0], [8000], k, v)
    p.evict(0, [0])
    got, want = run_multi(p, 0, [0], mq(27, 1, 4))
    assert max_err(got, want) <= TOL


def test_multi_query_errors():
    from quantized_decode_attention_append_amd import kvq
    p = Pair(cfg(max_seqs=9, n_layers=1))
    k, v = small_tokens(1, 40, 2, 256)
    p.append(0, [0, 1], [5, 35], k, v)
    for n_q in (0, 9):
        q = dev(mq(1, 1, max(n_q, 1))).view(1, max(n_q, 1), 16, 256)
        with pytest.raises(kvq.KvqError) as e:
            p.gpu.decode_attn_multi(0, [1], q[:, :n_q] if n_q == 0 else q)
        assert e.value.status == kvq.KVQ_E_INVALID
    with pytest.raises(kvq.KvqError) as e:        # 9 sequences x 8 queries > 64 entries
        p.gpu.decode_attn_multi(0, list(range(9)), dev(mq(2, 9, 8)).view(9, 8, 16, 256))
    assert e.value.status == kvq.KVQ_E_INVALID
    with pytest.raises(kvq.KvqError) as e:        # 5 positions, 6 queries
        p.gpu.decode_attn_multi(0, [0, 1], dev(mq(3, 2, 6)).view(2, 6, 16, 256))
    assert e.value.status == kvq.KVQ_E_STATE


@pytest.mark.parametrize("layout,tail_dtype,kvarn", [(0, 1, 0), (0, 2, 1), (0, 3, 0), (1, 1, 1), (1, 2, 0)])
def test_verify_and_roll_back_drafts(layout, tail_dtype, kvarn):
    """The draft-verification loop: append 1 + k tokens, decode them together, drop the rejected drafts with
    kvq_seq_truncate, then a fused decode step; slabs byte-exact and outputs within the tolerance every round."""
    p = Pair(cfg(layout=layout, tail_len=16, tail_slack=16, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=5, v_bits=3))
    seed = 500 + 10 * layout + tail_dtype + 3 * kvarn
    k, v = small_tokens(seed, 600, 2, 256)
    seqs = [0, 1]
    p.append(0, seqs, [120, 45], k[:165], v[:165])
    p.evict(0, seqs)
    off = 165
    for rnd, (n_q, keep) in enumerate(((8, (3, 8)), (5, (1, 5)), (8, (8, 2)), (2, (2, 1)))):
        p.append(0, seqs, [n_q, n_q], k[off:off + 2 * n_q], v[off:off + 2 * n_q])
        off += 2 * n_q
        got, want = run_multi(p, 0, seqs, mq(seed + rnd, 2, n_q))
        assert max_err(got, want) <= TOL, (rnd, max_err(got, want))
        new = [p.gpu.lengths(0, s)[0] - n_q + keep[i] for i, s in enumerate(seqs)]
        p.gpu.seq_truncate(0, seqs, new)
        p.ora.truncate(0, seqs, new)
        q = small_query(seed + 50 + rnd, 2, 16, 256)
        if layout == 0:
            got = p.gpu.decode_step(0, seqs, dev(k[off:off + 2]), dev(v[off:off + 2]), dev(q)).cpu().numpy()
            p.ora.append(0, seqs, [1, 1], k[off:off + 2], v[off:off + 2])
            p.ora.tail_evict(0, seqs)
            want = oracle.decode_reference(p.ora, 0, seqs, q)
            off += 2
        else:
            p.evict(0, seqs)
            got, want = p.decode(0, seqs, q)
        assert max_err(got, want) <= TOL, (rnd, max_err(got, want))
        for s in seqs:
            p.lengths_match(0, s)
            p.assert_slab_equal(0, s)


def test_truncate_errors_leave_the_cache_unchanged():
    from quantized_decode_attention_append_amd import kvq
    p = Pair(cfg(tail_len=16, tail_slack=16, tail_dtype=1))
    k, v = small_tokens(2, 100, 2, 256)
    p.append(0, [0, 1], [60, 30], k[:90], v[:90])
    p.evict(0, [0, 1])
    before = [p.gpu.lengths(0, s) for s in (0, 1)]
    for new, status in (([59, 31], kvq.KVQ_E_INVALID), ([40, 20], kvq.KVQ_E_STATE), ([-1, 30], kvq.KVQ_E_INVALID)):
        with pytest.raises(kvq.KvqError) as e:
            p.gpu.seq_truncate(0, [0, 1], new)
        assert e.value.status == status
        assert [p.gpu.lengths(0, s) for s in (0, 1)] == before


def _drafts(wl, layer, seq, n_q):
    """n_q decode-step tokens of a workload, appended as one chunk (the token being verified and its drafts)."""
    ks, vs = zip(*[W.decode_token(wl.cfg, layer, seq, st) for st in range(n_q)])
    return np.concatenate(ks), np.concatenate(vs)


def _workload_queries(wl, layer, n_seqs, n_q):
    return np.stack([np.stack([W.query(wl.cfg, layer, s, st) for st in range(n_q)]) for s in range(n_seqs)])


def test_multi_query_at_the_64k_workload_size():
    """T = 8 over layer 0 of the K6/V5 + bf16 tail workload at 65,536 positions, the size bench.py
    --config 2 --verify-queries 8 times."""
    from tests.test_gpu_fullsize import prefill_all
    wl = W.workload(2)
    p = Pair(dict(wl.cache_config(), n_layers=1))
    prefill_all(p, wl, 0)
    k, v = _drafts(wl, 0, 0, 8)
    p.append(0, [0], [8], k, v)
    got, want = run_multi(p, 0, [0], _workload_queries(wl, 0, 1, 8))
    assert max_err(got, want) <= TOL, max_err(got, want)


def test_multi_query_at_the_262k_workload_size():
    """T = 8 over layer 0 of the K6/V5 + q8_0 ring workload at 262,144 positions, the size bench.py --config 4
    --verify-queries 8 times: splits of ~64 tiles, the last of them crossing from body tiles into q8_0 ring tiles
    (the decode waves switch from the 6/5-bit decode to the 8-bit one within a split)."""
    from tests.test_gpu_fullsize import prefill_all
    wl = W.workload(4)
    p = Pair(dict(wl.cache_config(), n_layers=1))
    prefill_all(p, wl, 0)
    k, v = _drafts(wl, 0, 0, 8)
    p.append(0, [0], [8], k, v)
    got, want = run_multi(p, 0, [0], _workload_queries(wl, 0, 1, 8))
    assert max_err(got, want) <= TOL, max_err(got, want)


def test_multi_query_64_entries_at_the_eight_stream_workload_size():
    """8 streams x 8 queries (64 entries: ring segments planned outside the per-head budget) over layer 0 of the
    KVarN K4/V4 + bf16 tail workload at its full contexts (16k-64k), the size bench.py --config 3
    --verify-queries 8 times."""
    from tests.test_gpu_fullsize import prefill_all
    wl = W.workload(3)
    p = Pair(dict(wl.cache_config(), n_layers=1))
    prefill_all(p, wl, 0)
    seqs = list(range(wl.batch))
    for s in seqs:
        k, v = _drafts(wl, 0, s, 8)
        p.append(0, [s], [8], k, v)
    got, want = run_multi(p, 0, seqs, _workload_queries(wl, 0, wl.batch, 8))
    assert max_err(got, want) <= TOL, max_err(got, want)


@pytest.mark.parametrize("layout", [0, 1])
def test_multi_query_64_entries_with_bodies_of_thousands(layout):
    """8 sequences x 8 queries with bodies of 2k-8k positions, KVarN K4/V4 and a 1,024-position bf16 tail: the
    plan that gives the ring segments work-groups outside the per-head budget, with long body segments."""
    p = Pair(cfg(n_layers=1, max_seqs=8, capacity=8192 + 64, layout=layout, kvarn=1, k_bits=4, v_bits=4,
                 tail_len=1024, tail_slack=512, tail_dtype=1))
    rng = np.random.default_rng(31 + layout)
    lens = [int(x) for x in rng.integers(2048, 8192, size=8)]
    k, v = small_tokens(32 + layout, sum(lens) + 64, 2, 256,
                        scale=np.abs(np.random.default_rng(33).standard_t(3, size=(2, 2, 256))) + 0.05)
    p.append(0, list(range(8)), lens, k[:sum(lens)], v[:sum(lens)])
    p.evict(0, list(range(8)))
    p.append(0, list(range(8)), [8] * 8, k[sum(lens):], v[sum(lens):])
    got, want = run_multi(p, 0, list(range(8)), mq(34 + layout, 8, 8))
    assert max_err(got, want) <= TOL, max_err(got, want)
