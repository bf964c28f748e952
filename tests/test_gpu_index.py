"""GPU parity of the QSA indexer through the C ABI: pooled index keys byte-exact against the oracle for every
pooling ratio, and the chosen positions equal to the oracle's element by element (scores are defined bit for bit,
so the chosen set and its order are unique): ragged batches, sequences shorter than the budget, forced recent
positions, heavy ties, the full 262,144-position shape with a budget of 2,048; then sparse decode over the chosen
positions within 2e-3 of the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import TOL, Pair, dev, max_err
from workloads import small_query, small_tokens

pytestmark = pytest.mark.gpu


def icfg(**kw):
    c = dict(n_layers=2, max_seqs=4, capacity=6000, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=8, v_bits=8,
             kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, layout=1, index_dim=128, index_pool=4)
    c.update(kw)
    return c


def append_with_keys(p, layer, seq_ids, n_new, seed, dim=128, keys=None):
    k, v = small_tokens(seed, sum(n_new), p.cfg["n_kv_heads"], 256)
    p.append(layer, seq_ids, n_new, k, v)
    if keys is None:
        keys = W.bf16_bits(np.random.default_rng(seed).standard_normal((sum(n_new), dim), dtype=np.float32))
    p.gpu.index_write(layer, seq_ids, n_new, dev(keys))
    p.ora.index_write(layer, seq_ids, n_new, keys)
    return keys


def select_both(p, layer, seq_ids, q, budget, n_recent):
    got = p.gpu.index_select(layer, seq_ids, dev(q), budget, n_recent).cpu().numpy()
    want = p.ora.index_select(layer, seq_ids, q, budget, n_recent)
    return got, want


@pytest.mark.parametrize("pool", [1, 2, 4, 8, 16])
def test_index_keys_byte_exact(pool):
    p = Pair(icfg(index_dim=32 * pool, index_pool=pool, capacity=700))
    append_with_keys(p, 1, [0, 2], [300, 150], 10 + pool, dim=32 * pool)
    append_with_keys(p, 1, [2, 0], [1, 97], 20 + pool, dim=32 * pool)     # a second chunk, other order
    for s in (0, 2):
        p.lengths_match(1, s)
        p.assert_slab_equal(1, s)


@pytest.mark.parametrize("budget,n_recent", [(64, 0), (64, 16), (2048, 512), (256, 256), (1, 0), (1, 1)])
def test_index_select_matches_oracle(budget, n_recent):
    p = Pair(icfg())
    append_with_keys(p, 0, [0, 1, 2, 3], [5000, 1500, 40, 2100], 31)
    q = W.bf16_bits(np.random.default_rng(32).standard_normal((4, 32), dtype=np.float32))
    got, want = select_both(p, 0, [0, 1, 2, 3], q, budget, n_recent)
    np.testing.assert_array_equal(got, want)


def test_index_select_with_heavy_ties():
    """Keys and queries of few distinct values: many positions share a score, so the lower-position rule decides
    which of them are chosen."""
    p = Pair(icfg())
    rng = np.random.default_rng(41)
    keys = W.bf16_bits(rng.integers(-1, 2, size=(4500, 128)).astype(np.float32))
    append_with_keys(p, 0, [1, 3], [3000, 1500], 42, keys=keys)
    q = W.bf16_bits(rng.integers(-1, 2, size=(2, 32)).astype(np.float32))
    for budget, n_recent in ((100, 0), (700, 50), (2048, 512)):
        got, want = select_both(p, 0, [1, 3], q, budget, n_recent)
        np.testing.assert_array_equal(got, want)
    # every position the same score: the lowest positions win
    q0 = np.zeros((2, 32), dtype=np.uint16)
    got, want = select_both(p, 0, [1, 3], q0, 300, 10)
    np.testing.assert_array_equal(got, want)
    assert list(got[0][:290]) == list(range(290))


def test_index_select_empty_and_short_sequences():
    p = Pair(icfg())
    append_with_keys(p, 1, [1], [7], 51)
    q = W.bf16_bits(np.random.default_rng(52).standard_normal((2, 32), dtype=np.float32))
    got, want = select_both(p, 1, [0, 1], q, 16, 4)      # sequence 0 is empty
    np.testing.assert_array_equal(got, want)
    assert list(got[0]) == [-1] * 16 and list(got[1][:7]) == list(range(7))


def test_index_select_full_size():
    """The sparse workload's shape: 262,144 positions, budget 2,048 of which the 512 newest are forced."""
    cfg = icfg(n_layers=1, max_seqs=1, capacity=262144 + 64, n_kv_heads=1, n_q_heads=8)
    p = Pair(cfg)
    n = 262144
    for s in range(0, n, W.CHUNK):
        kk, vv = W.kv_tokens(5, 0, 0, s, W.CHUNK, n_kv_heads=1)
        p.append(0, [0], [W.CHUNK], kk, vv)
        keys = W.index_keys(5, 0, 0, s, W.CHUNK)
        p.gpu.index_write(0, [0], [W.CHUNK], dev(keys))
        p.ora.index_write(0, [0], [W.CHUNK], keys)
    p.assert_slab_equal(0, 0)
    for st in range(2):
        q = W.index_query(5, 0, 0, st)[None]
        got, want = select_both(p, 0, [0], q, 2048, 512)
        np.testing.assert_array_equal(got, want)


def test_sparse_decode_over_the_chosen_positions():
    p = Pair(icfg())
    append_with_keys(p, 0, [0, 2], [4000, 2500], 61)
    iq = W.bf16_bits(np.random.default_rng(62).standard_normal((2, 32), dtype=np.float32))
    pos = p.gpu.index_select(0, [0, 2], dev(iq), 1024, 128)
    want_pos = p.ora.index_select(0, [0, 2], iq, 1024, 128)
    np.testing.assert_array_equal(pos.cpu().numpy(), want_pos)
    q = small_query(63, 2, 16, 256)
    got = p.gpu.sparse_decode_attn(0, [0, 2], dev(q), pos).cpu().numpy()
    want = oracle.sparse_reference(p.ora, 0, [0, 2], q, want_pos)
    assert max_err(got, want) <= TOL


def test_index_errors():
    from quantized_decode_attention_append_amd import kvq
    p = Pair(icfg(index_dim=0, index_pool=0))
    k, v = small_tokens(1, 10, 2, 256)
    p.append(0, [0], [10], k, v)
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.index_write(0, [0], [10], dev(np.zeros((10, 128), dtype=np.uint16)))
    assert e.value.status == kvq.KVQ_E_INVALID
    p = Pair(icfg())
    p.append(0, [0], [10], k, v)
    with pytest.raises(kvq.KvqError) as e:                         # more keys than positions
        p.gpu.index_write(0, [0], [11], dev(np.zeros((11, 128), dtype=np.uint16)))
    assert e.value.status == kvq.KVQ_E_STATE
    q = dev(np.zeros((1, 32), dtype=np.uint16))
    with pytest.raises(kvq.KvqError) as e:                         # n_recent above the budget
        p.gpu.index_select(0, [0], q, 8, 9)
    assert e.value.status == kvq.KVQ_E_INVALID
    import torch
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.index_select(0, [0], q, 8, 0, workspace=small)
    assert e.value.status == kvq.KVQ_E_SIZE


def test_index_select_under_launch_timing():
    """With launch timing on, a select records one interval (scoring start to picking end) and still chooses the
    oracle's positions."""
    p = Pair(icfg())
    append_with_keys(p, 0, [0], [3000], 71)
    q = W.bf16_bits(np.random.default_rng(72).standard_normal((1, 32), dtype=np.float32))
    p.gpu.timing(True)
    got, want = select_both(p, 0, [0], q, 512, 64)
    ms, n = p.gpu.timing_read("index")
    p.gpu.timing(False)
    np.testing.assert_array_equal(got, want)
    assert n == 1 and ms > 0.0
