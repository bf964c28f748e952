"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Codes, scales, ring contents and KVarN scales must match byte for byte (whole slabs are compared, so
the layout of every region is checked too); attention outputs must be within 2e-3 absolute of the
oracle's fp64 result over the same dequantized values.
"""
import itertools

import numpy as np
import pytest

from tests.gpu_util import Pair, TOL, dev, max_err
from workloads import small_tokens, small_query, channel_scales

pytestmark = pytest.mark.gpu


def oracle_decode(p, layer, seq_ids, q):
    import oracle
    return oracle.decode_reference(p.ora, layer, seq_ids, q)


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=3, capacity=512, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=6,
             v_bits=5, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0)
    c.update(kw)
    return c


def scales(seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "loguniform":
        return (10.0 ** rng.uniform(-1, 1, size=(2, 2, 256))).astype(np.float32)
    if kind == "student":
        return np.abs(rng.standard_t(3, size=(2, 2, 256))).astype(np.float32)
    s = np.ones((2, 2, 256), dtype=np.float32)
    s[:, 0, [3, 77, 130, 201]] = 20.0
    return s


@pytest.mark.parametrize("nk,nv", list(itertools.product(range(2, 9), range(2, 9))))
def test_body_bytes_and_decode_no_tail(nk, nv):
    p = Pair(cfg(k_bits=nk, v_bits=nv))
    k, v = small_tokens(nk * 10 + nv, 300, 2, 256, scale=scales(nk, "outlier"))
    p.append(1, [2], [37], k[:37], v[:37])
    p.append(1, [2, 0], [64, 70], k[37:171], v[37:171])
    p.append(1, [2], [1], k[171:172], v[171:172])
    p.lengths_match(1, 2)
    p.assert_slab_equal(1, 2)
    p.assert_slab_equal(1, 0)
    q = small_query(nk + nv, 2, 16, 256)
    got, want = p.decode(1, [2, 0], q)
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
@pytest.mark.parametrize("kvarn", [0, 1])
def test_tail_ring_bytes_evict_and_decode(tail_dtype, kvarn):
    c = cfg(tail_len=64, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=6, v_bits=5)
    p = Pair(c)
    k, v = small_tokens(40 + tail_dtype + 2 * kvarn, 400, 2, 256, scale=scales(5, "student"))
    off = 0
    q = small_query(3, 1, 16, 256)
    # below the window, over the window, then decode-style steps, then a big chunk that overflows
    for n, ev in ((40, False), (30, False), (1, False), (50, True), (1, True), (1, True), (1, True), (150, False),
                  (3, True), (90, False)):
        p.append(0, [1], [n], k[off:off + n], v[off:off + n])
        off += n
        if ev:
            p.evict(0, [1])
        p.lengths_match(0, 1)
        p.assert_slab_equal(0, 1)
        got, want = p.decode(0, [1], q)
        assert max_err(got, want) <= TOL, (n, ev)


def test_kvarn_calibrates_on_first_chunk_only():
    c = cfg(kvarn=1, k_bits=4, v_bits=4)
    p = Pair(c)
    k, v = small_tokens(77, 200, 2, 256, scale=scales(7, "student"))
    p.append(0, [0, 1], [50, 20], k[:70], v[:70])
    p.append(0, [0], [130], k[70:200], v[70:200])
    for s in (0, 1):
        p.assert_slab_equal(0, s)
    got, want = p.decode(0, [0, 1], small_query(9, 2, 16, 256))
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("length", [1, 2, 31, 32, 33, 95, 129])
def test_decode_short_and_ragged(length):
    p = Pair(cfg(k_bits=8, v_bits=8))
    k, v = small_tokens(length, length, 2, 256)
    p.append(0, [0], [length], k, v)
    got, want = p.decode(0, [0], small_query(length, 1, 16, 256))
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
def test_ring_only_equals_lossless_or_q8(tail_dtype):
    # context below the window: a bf16 tail is lossless, an 8-bit ring behaves as q8_0 (pages' special cases),
    # an f16 tail holds the binary16 values
    p = Pair(cfg(tail_len=256, tail_slack=32, tail_dtype=tail_dtype))
    k, v = small_tokens(11, 200, 2, 256, scale=scales(2, "loguniform"))
    p.append(0, [0], [200], k, v)
    p.evict(0, [0])
    assert p.gpu.lengths(0, 0) == (200, 0)
    got, want = p.decode(0, [0], small_query(5, 1, 16, 256))
    assert max_err(got, want) <= TOL


def test_mixed_batch_lengths_and_heads():
    c = cfg(max_seqs=5, capacity=2048, tail_len=96, tail_slack=32, tail_dtype=1, k_bits=4, v_bits=4)
    p = Pair(c)
    lens = [1500, 7, 300, 96, 1]
    k, v = small_tokens(99, sum(lens), 2, 256, scale=scales(3, "loguniform"))
    p.append(0, [4, 0, 2, 1, 3], [lens[4], lens[0], lens[2], lens[1], lens[3]], k, v)
    p.evict(0, [0, 1, 2, 3, 4])
    for s in range(5):
        p.lengths_match(0, s)
        p.assert_slab_equal(0, s)
    got, want = p.decode(0, [3, 1, 0, 2, 4], small_query(8, 5, 16, 256))
    assert max_err(got, want) <= TOL


def test_softmax_scale_and_peaked_scores():
    p = Pair(cfg(k_bits=6, v_bits=5))
    k, v = small_tokens(5, 400, 2, 256, scale=scales(4, "loguniform"))
    p.append(0, [0], [400], k, v)
    q = small_query(6, 1, 16, 256, std=3.0)
    for sc in (0.0, 0.01, 0.5):
        got, want = p.decode(0, [0], q, sc)
        assert max_err(got, want) <= TOL, sc


def test_gqa_group_sizes():
    for hq in (2, 8, 16):
        p = Pair(cfg(n_q_heads=hq, k_bits=5, v_bits=4))
        k, v = small_tokens(hq, 100, 2, 256)
        p.append(0, [0], [100], k, v)
        got, want = p.decode(0, [0], small_query(hq, 1, hq, 256))
        assert max_err(got, want) <= TOL, hq


def test_errors_from_the_host():
    from quantized_decode_attention_append_amd import kvq
    p = Pair(cfg(capacity=64))
    k, v = small_tokens(1, 65, 2, 256)
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.decode_attn(0, [0], __import__("tests.gpu_util", fromlist=["dev"]).dev(small_query(0, 1, 16, 256)))
    assert e.value.status == kvq.KVQ_E_STATE
    p.append(0, [0], [64], k[:64], v[:64])
    from tests.gpu_util import dev
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.append(0, [0], [1], dev(k[64:]), dev(v[64:]))
    assert e.value.status == kvq.KVQ_E_CAPACITY
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.append(0, [0, 0], [0, 0], dev(k[:0]), dev(v[:0]))
    assert e.value.status == kvq.KVQ_E_INVALID
    import torch
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.decode_attn(0, [0], dev(small_query(0, 1, 16, 256)), workspace=ws)
    assert e.value.status == kvq.KVQ_E_SIZE


def test_workspace_reused_across_calls_and_allocations():
    # many calls on one workspace, with unrelated allocations in between, must all be right
    import torch
    p = Pair(cfg(k_bits=4, v_bits=4, capacity=4096))
    k, v = small_tokens(3, 3000, 2, 256)
    p.append(0, [0], [3000], k, v)
    ws = p.gpu.workspace(1, 3000)
    for i in range(6):
        junk = torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda")
        q = small_query(100 + i, 1, 16, 256)
        from tests.gpu_util import dev
        import oracle
        got = p.gpu.decode_attn(0, [0], dev(q), workspace=ws).cpu().numpy()
        want = oracle.decode_reference(p.ora, 0, [0], q)
        assert max_err(got, want) <= TOL, i
        del junk



@pytest.mark.parametrize("tail_dtype,kvarn", [(1, 0), (2, 0), (1, 1), (0, 0), (3, 0)])
def test_append_evict_matches_append_then_evict(tail_dtype, kvarn):
    """kvq_append_evict against the oracle doing the two calls: decode steps (one launch), a batch with an
    empty sequence, a chunk that evicts its own rows and the first (calibrating) append (two launches)."""
    tail = 64 if tail_dtype else 0
    c = cfg(tail_len=tail, tail_slack=32 if tail else 0, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=5, v_bits=4)
    p = Pair(c)
    k, v = small_tokens(70 + tail_dtype + 3 * kvarn, 600, 2, 256, scale=scales(9, "loguniform"))
    q = small_query(11, 2, 16, 256)
    off = 0

    def step(seq_ids, ns):
        nonlocal off
        tot = sum(ns)
        p.gpu.append_evict(1, seq_ids, ns, dev(k[off:off + tot]), dev(v[off:off + tot]))
        p.ora.append(1, seq_ids, ns, k[off:off + tot], v[off:off + tot])
        p.ora.tail_evict(1, seq_ids)
        off += tot
        for s in seq_ids:
            p.lengths_match(1, s)
            p.assert_slab_equal(1, s)

    p.gpu.timing(True)             # counts the launches of each kernel kind
    step([0, 2], [90, 5])          # first append: calibration, body writes, ring overflow
    for _ in range(4):
        step([0, 2], [1, 1])       # decode steps
    step([2, 0], [0, 1])           # one sequence without a token
    step([0], [100])               # a chunk longer than the window evicts rows of its own
    step([0, 2], [1, 3])
    fused = p.gpu.timing_read("append_evict")[1]
    p.gpu.timing(False)
    assert fused == (6 if tail_dtype else 0), fused   # the decode-style steps took the single launch
    got, want = p.decode(1, [0, 2], q)
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("tail_dtype,kvarn,n_seqs", [(1, 0, 1), (2, 0, 2), (1, 1, 3), (2, 1, 1), (3, 1, 2)])
def test_decode_step_matches_append_evict_decode(tail_dtype, kvarn, n_seqs):
    """kvq_decode_step (the append and evict written inside the decode launch) against the oracle doing append,
    evict and decode: ring bytes, body bytes and outputs after every step, for sequences whose ring is below the
    window (no requantization yet), just filling it, and in steady state."""
    c = cfg(tail_len=64, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=6, v_bits=5, capacity=1024)
    p = Pair(c)
    rng_seed = 90 + tail_dtype + 2 * kvarn + 5 * n_seqs
    k, v = small_tokens(rng_seed, 1200, 2, 256, scale=scales(7, "loguniform"))
    seqs = list(range(n_seqs))
    off = 0
    # a prefill below and one above the window for the first sequence, shorter ones for the others
    for i, n in zip(seqs, (150, 40, 63)):
        p.append(1, [i], [n], k[off:off + n], v[off:off + n])
        off += n
    p.evict(1, seqs)
    p.gpu.timing(True)
    for step in range(6):
        kk, vv = k[off:off + n_seqs], v[off:off + n_seqs]
        off += n_seqs
        q = small_query(rng_seed + step, n_seqs, 16, 256)
        got = p.gpu.decode_step(1, seqs, dev(kk), dev(vv), dev(q)).cpu().numpy()
        p.ora.append(1, seqs, [1] * n_seqs, kk, vv)
        p.ora.tail_evict(1, seqs)
        want = oracle_decode(p, 1, seqs, q)
        for i in seqs:
            p.lengths_match(1, i)
            p.assert_slab_equal(1, i)
        assert max_err(got, want) <= TOL, f"step {step}: {max_err(got, want):.3e}"
    separate = p.gpu.timing_read("append")[1] + p.gpu.timing_read("append_evict")[1]
    p.gpu.timing(False)
    assert separate == 0, separate   # every step ran in the decode launch


def test_largest_batch_of_64_sequences():
    """A call over the largest batch (64 sequences, ragged lengths 1..130): one append, evict, decode, and decode
    steps (more sequences than one fused step launch takes: the step falls back to its separate calls)."""
    import oracle
    c = cfg(max_seqs=64, capacity=256, tail_len=32, tail_slack=32, tail_dtype=1, k_bits=4, v_bits=3, n_layers=1)
    p = Pair(c)
    rng = np.random.default_rng(64)
    lens = [int(x) for x in rng.integers(1, 131, size=64)]
    k, v = small_tokens(640, sum(lens) + 64 * 3, 2, 256)
    seqs = list(range(64))
    p.append(0, seqs, lens, k[:sum(lens)], v[:sum(lens)])
    p.evict(0, seqs)
    for s in (0, 17, 63):
        p.lengths_match(0, s)
        p.assert_slab_equal(0, s)
    q = small_query(64, 64, 16, 256)
    got, want = p.decode(0, seqs, q)
    assert max_err(got, want) <= TOL
    off = sum(lens)
    for st in range(2):
        kk, vv = k[off:off + 64], v[off:off + 64]
        off += 64
        q = small_query(65 + st, 64, 16, 256)
        got = p.gpu.decode_step(0, seqs, dev(kk), dev(vv), dev(q)).cpu().numpy()
        p.ora.append(0, seqs, [1] * 64, kk, vv)
        p.ora.tail_evict(0, seqs)
        want = oracle.decode_reference(p.ora, 0, seqs, q)
        assert max_err(got, want) <= TOL, st
        for s in (5, 40, 63):
            p.lengths_match(0, s)
            p.assert_slab_equal(0, s)


def test_seq_reset_reuses_a_slab_like_a_fresh_sequence():
    """kvq_seq_reset: the sequence's slab is zeroed and its lengths and KVarN calibration forgotten (the oracle's
    fresh state); a new token stream then recalibrates and matches a fresh oracle sequence byte for byte; other
    sequences and layers are untouched."""
    c = cfg(kvarn=1, tail_len=64, tail_slack=32, tail_dtype=1, k_bits=5, v_bits=4)
    p = Pair(c)
    k, v = small_tokens(90, 240, 2, 256, scale=scales(3, "student"))
    k2, v2 = small_tokens(91, 150, 2, 256, scale=scales(4, "loguniform"))
    p.append(0, [0, 1], [150, 90], k, v)
    p.append(1, [0], [60], k[:60], v[:60])
    p.evict(0, [0, 1])
    p.gpu.seq_reset(0, [0])
    p.ora.state.pop((0, 0), None)
    assert p.gpu.lengths(0, 0) == (0, 0)
    for layer, seq in ((0, 0), (0, 1), (1, 0)):
        p.assert_slab_equal(layer, seq)
    p.append(0, [0], [120], k2[:120], v2[:120])
    p.evict(0, [0])
    p.lengths_match(0, 0)
    p.assert_slab_equal(0, 0)
    got, want = p.decode(0, [0, 1], small_query(12, 2, 16, 256))
    assert max_err(got, want) <= TOL
    # every layer at once
    p.gpu.seq_reset(-1, [0])
    for layer in (0, 1):
        p.ora.state.pop((layer, 0), None)
        assert p.gpu.lengths(layer, 0) == (0, 0)
        p.assert_slab_equal(layer, 0)
    p.assert_slab_equal(0, 1)


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
def test_decode_steps_across_ring_wraparound(tail_dtype):
    """Many fused decode steps on a small ring (R = 64 slots): ring slots wrap around several times, the row
    leaving the window and the appended row sit in every slot position, and the body grows tile by tile."""
    import oracle
    c = cfg(tail_len=32, tail_slack=32, tail_dtype=tail_dtype, k_bits=6, v_bits=5, capacity=512, n_layers=1)
    p = Pair(c)
    k, v = small_tokens(120 + tail_dtype, 300, 2, 256, scale=scales(6, "loguniform"))
    p.append(0, [0, 1], [40, 7], k[:47], v[:47])
    p.evict(0, [0, 1])
    off = 47
    for step in range(150):
        kk, vv = k[off:off + 2], v[off:off + 2]
        off = 47 + (off - 47 + 2) % 250   # reuse the token pool
        q = small_query(300 + step, 2, 16, 256)
        got = p.gpu.decode_step(0, [0, 1], dev(kk), dev(vv), dev(q)).cpu().numpy()
        p.ora.append(0, [0, 1], [1, 1], kk, vv)
        p.ora.tail_evict(0, [0, 1])
        if step % 25 == 24 or step < 3:
            want = oracle.decode_reference(p.ora, 0, [0, 1], q)
            assert max_err(got, want) <= TOL, step
            for s in (0, 1):
                p.lengths_match(0, s)
                p.assert_slab_equal(0, s)


@pytest.mark.parametrize("hk,hq", [(1, 4), (4, 32), (8, 8), (3, 21)])
def test_kv_head_counts(hk, hq):
    """Other numbers of KV heads (and groups of 1 to 8 query heads): bytes, decode and a fused decode step in
    the tile layout; bytes and sparse decode, plain and fused, in the row layout."""
    import oracle
    import torch
    c = cfg(n_kv_heads=hk, n_q_heads=hq, tail_len=64, tail_slack=32, tail_dtype=1, k_bits=6, v_bits=5)
    p = Pair(c)
    k, v = small_tokens(200 + hk, 300, hk, 256)
    p.append(0, [0, 1], [180, 60], k[:240], v[:240])
    p.evict(0, [0, 1])
    for s in (0, 1):
        p.assert_slab_equal(0, s)
    q = small_query(hk, 2, hq, 256)
    got, want = p.decode(0, [0, 1], q)
    assert max_err(got, want) <= TOL
    got = p.gpu.decode_step(0, [0, 1], dev(k[240:242]), dev(v[240:242]), dev(q)).cpu().numpy()
    p.ora.append(0, [0, 1], [1, 1], k[240:242], v[240:242])
    p.ora.tail_evict(0, [0, 1])
    assert max_err(got, oracle.decode_reference(p.ora, 0, [0, 1], q)) <= TOL
    for s in (0, 1):
        p.assert_slab_equal(0, s)
    r = Pair(cfg(n_kv_heads=hk, n_q_heads=hq, k_bits=8, v_bits=8, layout=1))
    r.append(0, [0], [200], k[:200], v[:200])
    r.assert_slab_equal(0, 0)
    rng = np.random.default_rng(hk)
    pos = rng.choice(200, size=70, replace=False).astype(np.int32)[None]
    got, want = r.sparse(0, [0], q[:1], pos)
    assert max_err(got, want) <= TOL
    pos2 = np.concatenate([[200], rng.choice(200, size=69, replace=False)]).astype(np.int32)[None]
    got = r.gpu.sparse_decode_step(0, [0], dev(k[200:201]), dev(v[200:201]), dev(q[:1]),
                                   torch.from_numpy(pos2).to("cuda")).cpu().numpy()
    r.ora.append(0, [0], [1], k[200:201], v[200:201])
    assert max_err(got, oracle.sparse_reference(r.ora, 0, [0], q[:1], pos2)) <= TOL
    r.assert_slab_equal(0, 0)


RING_WIDTHS = [(2, 5, 1, 0), (3, 7, 2, 1), (4, 2, 3, 0), (5, 8, 1, 1), (6, 3, 2, 0), (7, 6, 3, 1), (8, 4, 1, 1)]


@pytest.mark.parametrize("nk,nv,tail_dtype,kvarn", RING_WIDTHS)
def test_ring_requantized_into_every_body_width(nk, nv, tail_dtype, kvarn):
    """Ring rows leaving the window are requantized into bodies of every K and V width (each of 2..8 bits once
    on each side, over all three ring kinds, with and without KVarN): after a prefill past the window, through
    fused decode steps, and through a separate append of a chunk larger than the window followed by an evict."""
    c = cfg(tail_len=32, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn, k_bits=nk, v_bits=nv, capacity=512)
    p = Pair(c)
    seed = 300 + 10 * nk + nv
    k, v = small_tokens(seed, 300, 2, 256, scale=scales(nk, "student" if kvarn else "loguniform"))
    seqs = [0, 2]
    p.append(0, seqs, [100, 45], k[:145], v[:145])
    p.evict(0, seqs)
    off = 145
    for i in seqs:
        p.lengths_match(0, i)
        p.assert_slab_equal(0, i)
    for step in range(4):
        kk, vv = k[off:off + 2], v[off:off + 2]
        off += 2
        q = small_query(seed + step, 2, 16, 256)
        got = p.gpu.decode_step(0, seqs, dev(kk), dev(vv), dev(q)).cpu().numpy()
        p.ora.append(0, seqs, [1, 1], kk, vv)
        p.ora.tail_evict(0, seqs)
        want = oracle_decode(p, 0, seqs, q)
        for i in seqs:
            p.lengths_match(0, i)
            p.assert_slab_equal(0, i)
        assert max_err(got, want) <= TOL, f"step {step}: {max_err(got, want):.3e}"
    p.append(0, [2], [70], k[off:off + 70], v[off:off + 70])
    p.evict(0, [2])
    p.lengths_match(0, 2)
    p.assert_slab_equal(0, 2)
    got, want = p.decode(0, seqs, small_query(seed + 9, 2, 16, 256))
    assert max_err(got, want) <= TOL
