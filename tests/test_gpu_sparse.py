"""GPU parity of the row layout and of sparse (gather) decode, through the C ABI, against the oracle.

A row-layout cache must hold exactly the oracle's bytes; dense decode of a row-layout cache and sparse
decode over a position list must be within 2e-3 of the oracle's fp64 attention. Invariants from the
definition of attention: a list holding every position once equals dense decode, in any order; a list
over a cache equals dense decode over a cache holding only the listed tokens.
"""
import itertools

import numpy as np
import pytest

from tests.gpu_util import Pair, TOL, max_err, dev
from workloads import small_tokens, small_query

pytestmark = pytest.mark.gpu


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=3, capacity=512, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=8,
             v_bits=8, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, layout=1)
    c.update(kw)
    return c


def outlier_scale():
    s = np.ones((2, 2, 256), dtype=np.float32)
    s[:, 0, [5, 99, 140, 250]] = 20.0
    return s


@pytest.mark.parametrize("nk,nv", list(itertools.product(range(2, 9), range(2, 9))))
def test_rows_bytes_dense_and_sparse(nk, nv):
    p = Pair(cfg(k_bits=nk, v_bits=nv))
    k, v = small_tokens(500 + nk * 10 + nv, 300, 2, 256, scale=outlier_scale())
    p.append(1, [2], [37], k[:37], v[:37])
    p.append(1, [2, 0], [64, 70], k[37:171], v[37:171])
    p.lengths_match(1, 2)
    p.assert_slab_equal(1, 2)
    p.assert_slab_equal(1, 0)
    q = small_query(nk * nv, 2, 16, 256)
    got, want = p.decode(1, [2, 0], q)
    assert max_err(got, want) <= TOL
    rng = np.random.default_rng(nk * 7 + nv)
    pos = np.stack([rng.choice(101, size=40, replace=False), rng.choice(70, size=40, replace=False)])
    got, want = p.sparse(1, [2, 0], q, pos)
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
@pytest.mark.parametrize("kvarn", [0, 1])
def test_rows_tail_ring_evict_dense_and_sparse(tail_dtype, kvarn):
    c = cfg(tail_len=64, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=6, v_bits=5)
    p = Pair(c)
    k, v = small_tokens(600 + tail_dtype + 2 * kvarn, 400, 2, 256, scale=outlier_scale())
    q = small_query(13, 1, 16, 256)
    off = 0
    rng = np.random.default_rng(tail_dtype * 3 + kvarn)
    for n, ev in ((40, False), (50, True), (1, True), (150, False), (3, True), (90, False)):
        p.append(0, [1], [n], k[off:off + n], v[off:off + n])
        off += n
        if ev:
            p.evict(0, [1])
        p.lengths_match(0, 1)
        p.assert_slab_equal(0, 1)
        got, want = p.decode(0, [1], q)
        assert max_err(got, want) <= TOL, (n, ev)
        # a list that mixes body and ring rows
        pos = rng.choice(off, size=min(off, 77), replace=False)[None]
        got, want = p.sparse(0, [1], q, pos)
        assert max_err(got, want) <= TOL, (n, ev)


def test_sparse_over_every_position_equals_dense_in_any_order():
    p = Pair(cfg(k_bits=5, v_bits=4, capacity=2048))
    k, v = small_tokens(7, 1500, 2, 256)
    p.append(0, [0], [1500], k, v)
    q = small_query(21, 1, 16, 256, std=2.0)
    dense, want = p.decode(0, [0], q)
    assert max_err(dense, want) <= TOL
    for seed in range(3):
        perm = np.random.default_rng(seed).permutation(1500)[None]
        got, _ = p.sparse(0, [0], q, perm)
        assert max_err(got, want) <= TOL, seed
        assert float(np.max(np.abs(got - dense))) <= 1e-4, seed


def test_sparse_equals_dense_over_a_cache_of_the_listed_tokens():
    # no ring: each row depends on its own token only, so a cache holding just the listed tokens
    # (appended in list order) attends over the same rows
    c = cfg(k_bits=8, v_bits=8, capacity=4096, max_seqs=1)
    p = Pair(c)
    k, v = small_tokens(31, 4000, 2, 256)
    p.append(0, [0], [4000], k, v)
    rng = np.random.default_rng(5)
    pos = np.concatenate([np.arange(3600, 4000), rng.choice(3600, size=624, replace=False)])
    q = small_query(41, 1, 16, 256)
    got, _ = p.sparse(0, [0], q, pos[None])
    small = Pair(cfg(k_bits=8, v_bits=8, capacity=1024, max_seqs=1))
    small.append(0, [0], [len(pos)], k[pos], v[pos])
    ref, want = small.decode(0, [0], q)
    assert max_err(ref, want) <= TOL
    assert max_err(got, want) <= TOL
    assert float(np.max(np.abs(got - ref))) <= 1e-4


def test_sparse_skips_out_of_range_and_counts_repeats():
    p = Pair(cfg(k_bits=4, v_bits=4))
    k, v = small_tokens(9, 200, 2, 256)
    p.append(0, [0, 1], [150, 50], k, v)
    q = small_query(3, 2, 16, 256)
    pos = np.array([[-1, 3, 3, 149, 150, 7000, 20, 20, 20, 0],
                    [49, 50, 51, -5, 0, 1, 1, 2, 48, 10]], dtype=np.int32)
    got, want = p.sparse(0, [0, 1], q, pos)
    assert max_err(got, want) <= TOL
    none = np.array([[-1, 150, 151, 99999]], dtype=np.int32)
    got, want = p.sparse(0, [0], q[:1], none)
    assert np.all(got == 0.0) and np.all(want == 0.0)


def test_sparse_budget_one_and_mixed_batch():
    p = Pair(cfg(k_bits=6, v_bits=5, max_seqs=3, capacity=1024, tail_len=64, tail_slack=64, tail_dtype=2))
    k, v = small_tokens(11, 1200, 2, 256)
    p.append(0, [2, 0, 1], [700, 5, 300], k[:1005], v[:1005])
    p.evict(0, [0, 1, 2])
    q = small_query(17, 3, 16, 256)
    got, want = p.sparse(0, [0, 1, 2], q, np.array([[4], [299], [0]], dtype=np.int32))
    assert max_err(got, want) <= TOL
    rng = np.random.default_rng(1)
    pos = np.stack([rng.choice(5, size=5, replace=False).tolist() + [0] * 295,
                    rng.choice(300, size=300, replace=False), rng.choice(700, size=300, replace=False)])
    got, want = p.sparse(0, [0, 1, 2], q, pos.astype(np.int32))
    assert max_err(got, want) <= TOL


def test_sparse_needs_the_row_layout():
    from quantized_decode_attention_append_amd import kvq
    import torch
    p = Pair(cfg(layout=0))
    k, v = small_tokens(2, 64, 2, 256)
    p.append(0, [0], [64], k, v)
    pos = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.sparse_decode_attn(0, [0], dev(small_query(0, 1, 16, 256)), pos)
    assert e.value.status == kvq.KVQ_E_INVALID
    # the fused step checks the same before it appends anything
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.sparse_decode_step(0, [0], dev(k[:1]), dev(v[:1]), dev(small_query(0, 1, 16, 256)), pos)
    assert e.value.status == kvq.KVQ_E_INVALID
    assert p.gpu.lengths(0, 0) == (64, 64)


def test_sparse_decode_step_errors_leave_the_cache_unchanged():
    from quantized_decode_attention_append_amd import kvq
    import torch
    p = Pair(cfg(capacity=64))
    k, v = small_tokens(3, 65, 2, 256)
    p.append(0, [0], [64], k[:64], v[:64])
    q = dev(small_query(1, 1, 16, 256))
    pos = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:   # full: the append is refused
        p.gpu.sparse_decode_step(0, [0], dev(k[64:]), dev(v[64:]), q, pos)
    assert e.value.status == kvq.KVQ_E_CAPACITY
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    p2 = Pair(cfg())
    p2.append(0, [0], [64], k[:64], v[:64])
    with pytest.raises(kvq.KvqError) as e:   # workspace too small: reported before the launch
        p2.gpu.sparse_decode_step(0, [0], dev(k[64:]), dev(v[64:]), q, pos, workspace=ws)
    assert e.value.status == kvq.KVQ_E_SIZE
    assert p.gpu.lengths(0, 0) == (64, 64) and p2.gpu.lengths(0, 0) == (64, 64)
    p2.assert_slab_equal(0, 0)


@pytest.mark.parametrize("nk,nv,kvarn,tail_dtype,n_seqs", [(8, 8, 0, 0, 1), (6, 5, 1, 0, 2), (3, 7, 0, 0, 3),
                                                          (4, 4, 0, 1, 1), (8, 8, 1, 0, 1), (6, 5, 0, 3, 2)])
def test_sparse_decode_step_matches_append_then_sparse(nk, nv, kvarn, tail_dtype, n_seqs):
    """kvq_sparse_decode_step against the oracle doing the append and then sparse decode: body bytes and
    outputs after every step. Without a ring (and calibrated KVarN scales) the new rows are written inside the
    gather launch, also by work-groups whose range lists the new position (the list holds it at varying
    places, or not at all); with a ring, or before KVarN calibration, the calls run in turn."""
    c = cfg(k_bits=nk, v_bits=nv, kvarn=kvarn, tail_dtype=tail_dtype, tail_len=64 if tail_dtype else 0,
            tail_slack=32 if tail_dtype else 0, capacity=1024)
    p = Pair(c)
    k, v = small_tokens(700 + nk * 10 + nv + kvarn, 900, 2, 256, scale=outlier_scale())
    seqs = list(range(n_seqs))
    off = 0
    for i, n in zip(seqs, (300, 150, 125)):
        p.append(0, [i], [n], k[off:off + n], v[off:off + n])
        off += n
    rng = np.random.default_rng(nk + 10 * nv + 100 * kvarn)
    p.gpu.timing(True)
    for step in range(5):
        kk, vv = k[off:off + n_seqs], v[off:off + n_seqs]
        off += n_seqs
        lens = [p.gpu.lengths(0, i)[0] + 1 for i in seqs]
        budget = 120   # two list ranges per KV head: the new position falls in either, or in none
        pos = []
        for i, n in enumerate(lens):
            recent = np.arange(n - 16, n)
            rest = rng.choice(n - 16, size=budget - 16, replace=False)
            lst = np.concatenate([rest, recent]) if step % 2 else np.concatenate([recent, rest])
            if step == 3 and i == 0:
                lst = rest[:budget]   # the new position not listed: still appended
                lst = np.concatenate([lst, rng.choice(n - 16, size=budget - len(lst), replace=False)])
            pos.append(lst)
        pos = np.stack(pos).astype(np.int32)
        q = small_query(50 + step, n_seqs, 16, 256)
        import torch
        got = p.gpu.sparse_decode_step(0, seqs, dev(kk), dev(vv), dev(q), torch.from_numpy(pos).to("cuda")).cpu().numpy()
        p.ora.append(0, seqs, [1] * n_seqs, kk, vv)
        import oracle
        want = oracle.sparse_reference(p.ora, 0, seqs, q, pos)
        for i in seqs:
            p.lengths_match(0, i)
            p.assert_slab_equal(0, i)
        assert max_err(got, want) <= TOL, f"step {step}: {max_err(got, want):.3e}"
    appends = p.gpu.timing_read("append")[1]
    p.gpu.timing(False)
    if tail_dtype == 0:
        assert appends == 0, appends   # every step's append ran in the gather launch
    else:
        assert appends > 0


def test_sparse_largest_batch_and_fused_step():
    """64 sequences in one sparse call and one fused sparse step (the new rows written in the gather launch)."""
    import oracle
    import torch
    p = Pair(cfg(max_seqs=64, capacity=256, n_layers=1, k_bits=5, v_bits=6))
    rng = np.random.default_rng(640)
    lens = [int(x) for x in rng.integers(40, 200, size=64)]
    k, v = small_tokens(641, sum(lens) + 64, 2, 256)
    seqs = list(range(64))
    p.append(0, seqs, lens, k[:sum(lens)], v[:sum(lens)])
    q = small_query(66, 64, 16, 256)
    pos = np.stack([rng.choice(n, size=32, replace=False) for n in lens]).astype(np.int32)
    got, want = p.sparse(0, seqs, q, pos)
    assert max_err(got, want) <= TOL
    kk, vv = k[sum(lens):], v[sum(lens):]
    pos = np.stack([np.concatenate([[n], rng.choice(n, size=31, replace=False)]) for n in lens]).astype(np.int32)
    got = p.gpu.sparse_decode_step(0, seqs, dev(kk), dev(vv), dev(q), torch.from_numpy(pos).to("cuda")).cpu().numpy()
    p.ora.append(0, seqs, [1] * 64, kk, vv)
    want = oracle.sparse_reference(p.ora, 0, seqs, q, pos)
    assert max_err(got, want) <= TOL
    for s in (0, 31, 63):
        p.lengths_match(0, s)
        p.assert_slab_equal(0, s)


def test_many_fused_sparse_steps():
    """100 fused sparse steps (the appended row written inside the gather launch each time), lists of newest +
    drawn positions of varying budget placement; bytes and outputs checked along the way."""
    import oracle
    import torch
    p = Pair(cfg(k_bits=6, v_bits=4, capacity=512, n_layers=1, max_seqs=2, kvarn=1))
    k, v = small_tokens(777, 400, 2, 256, scale=outlier_scale())
    p.append(0, [0, 1], [100, 33], k[:133], v[:133])
    rng = np.random.default_rng(777)
    off = 133
    for step in range(100):
        kk, vv = k[off:off + 2], v[off:off + 2]
        off += 2
        lens = [p.gpu.lengths(0, s)[0] + 1 for s in (0, 1)]
        budget = 24
        pos = np.stack([np.concatenate([np.arange(n - 8, n), rng.choice(n - 8, size=budget - 8, replace=False)])
                        [rng.permutation(budget)] for n in lens]).astype(np.int32)
        q = small_query(900 + step, 2, 16, 256)
        got = p.gpu.sparse_decode_step(0, [0, 1], dev(kk), dev(vv), dev(q), torch.from_numpy(pos).to("cuda")).cpu().numpy()
        p.ora.append(0, [0, 1], [1, 1], kk, vv)
        if step % 20 == 19 or step < 2:
            want = oracle.sparse_reference(p.ora, 0, [0, 1], q, pos)
            assert max_err(got, want) <= TOL, step
            for s in (0, 1):
                p.lengths_match(0, s)
                p.assert_slab_equal(0, s)


def test_long_lists_take_several_steps_per_wave():
    """Lists long enough that every wave takes several 16-entry steps (the split count is capped by the
    work-group budget): dense decode of a 40,000-position row-layout cache with a q8_0 ring, and a fused
    sparse step over a 30,000-entry list that holds the new position near its end."""
    import oracle
    import torch
    c = cfg(k_bits=6, v_bits=5, capacity=40960, n_layers=1, max_seqs=1, tail_len=64, tail_slack=64, tail_dtype=2)
    p = Pair(c)
    n = 40000
    for s0 in range(0, n, 8000):
        k, v = small_tokens(900 + s0 // 8000, 8000, 2, 256)
        p.append(0, [0], [8000], k, v)
    p.evict(0, [0])
    p.lengths_match(0, 0)
    q = small_query(77, 1, 16, 256)
    got, want = p.decode(0, [0], q)
    assert max_err(got, want) <= TOL
    c2 = cfg(k_bits=8, v_bits=8, capacity=40960, n_layers=1, max_seqs=1)
    p2 = Pair(c2)
    k, v = small_tokens(950, 32001, 2, 256)
    p2.append(0, [0], [32000], k[:32000], v[:32000])
    rng = np.random.default_rng(951)
    pos = rng.choice(32000, size=30000, replace=False).astype(np.int32)
    pos[-5] = 32000   # the appended position
    got = p2.gpu.sparse_decode_step(0, [0], dev(k[32000:]), dev(v[32000:]), dev(q),
                                    torch.from_numpy(pos[None].copy()).to("cuda")).cpu().numpy()
    p2.ora.append(0, [0], [1], k[32000:], v[32000:])
    want = oracle.sparse_reference(p2.ora, 0, [0], q, pos[None])
    assert max_err(got, want) <= TOL
    p2.lengths_match(0, 0)


@pytest.mark.parametrize("nk,nv,tail_dtype,kvarn", [(2, 5, 1, 0), (3, 7, 2, 1), (4, 2, 3, 0), (5, 8, 1, 1),
                                                    (6, 3, 2, 0), (7, 6, 3, 1), (8, 4, 1, 1)])
def test_rows_ring_requantized_into_every_body_width(nk, nv, tail_dtype, kvarn):
    """Row layout: ring rows leaving the window are requantized into body rows of every K and V width (each of
    2..8 bits once on each side, over all three ring kinds, with and without KVarN); dense decode through the
    gather and sparse lists that mix body and ring rows agree with the oracle after every step."""
    p = Pair(cfg(tail_len=32, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=nk, v_bits=nv))
    k, v = small_tokens(700 + 10 * nk + nv, 300, 2, 256, scale=outlier_scale())
    rng = np.random.default_rng(nk * 11 + nv)
    off = 0
    for n, ev in ((20, False), (60, True), (1, True), (1, True), (70, False), (2, True)):
        p.append(0, [2], [n], k[off:off + n], v[off:off + n])
        off += n
        if ev:
            p.evict(0, [2])
        p.lengths_match(0, 2)
        p.assert_slab_equal(0, 2)
        q = small_query(off, 1, 16, 256)
        got, want = p.decode(0, [2], q)
        assert max_err(got, want) <= TOL, (n, ev)
        pos = rng.choice(off, size=min(off, 45), replace=False)[None]
        got, want = p.sparse(0, [2], q, pos)
        assert max_err(got, want) <= TOL, (n, ev)
