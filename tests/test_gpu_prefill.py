"""GPU parity of chunked prefill attention (kvq_prefill_attn: append a chunk, then causal attention of its queries
over the cache as it then stands) through the C ABI, against the oracle's fp64 result over the same dequantized
values: within 2e-3 absolute, every ring kind and KVarN, ragged chunks of several sequences (one of them empty),
query blocks that straddle the body / ring boundary, and the slabs byte-exact with the oracle's after each
chunk."""
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


def run_prefill(p, layer, seqs, n_new, k, v, q, rows=None):
    print(f"prefill layer {layer} seqs {seqs} n_new {n_new}", flush=True)
    got = p.gpu.prefill_attn(layer, seqs, n_new, dev(k), dev(v), dev(q)).cpu().numpy()
    p.ora.append(layer, seqs, n_new, k, v)
    want = oracle.prefill_reference(p.ora, layer, seqs, n_new, q, rows)
    return (got if rows is None else got[rows]), want


CHUNKS = ([100, 37], [0, 70], [300, 5], [1, 1], [64, 9])


@pytest.mark.parametrize("tail_dtype,kvarn,k_bits,v_bits,evict", [
    (0, 0, 6, 5, 0), (1, 0, 6, 5, 1), (2, 1, 6, 5, 1), (3, 0, 4, 4, 0), (1, 1, 2, 8, 0), (2, 0, 8, 3, 0),
    (0, 1, 3, 7, 0), (3, 1, 5, 2, 1), (2, 0, 7, 6, 0)])
def test_prefill_chunks_match_oracle(tail_dtype, kvarn, k_bits, v_bits, evict):
    tail = dict(tail_len=64, tail_slack=32, tail_dtype=tail_dtype) if tail_dtype else {}
    p = Pair(cfg(kvarn=kvarn, k_bits=k_bits, v_bits=v_bits, **tail))
    seed = 7 * tail_dtype + 3 * kvarn + k_bits + 11 * v_bits
    k, v = small_tokens(seed, sum(map(sum, CHUNKS)), 2, 256)
    q = small_query(seed + 1, sum(map(sum, CHUNKS)), 16, 256)
    off = 0
    for n_new in CHUNKS:
        n = sum(n_new)
        got, want = run_prefill(p, 1, [0, 2], n_new, k[off:off + n], v[off:off + n], q[off:off + n])
        assert max_err(got, want) <= TOL, (n_new, max_err(got, want))
        off += n
        if evict:
            p.evict(1, [0, 2])
        for s in (0, 2):
            p.lengths_match(1, s)
            p.assert_slab_equal(1, s)


@pytest.mark.parametrize("hq", [2, 8])
def test_prefill_group_sizes(hq):
    """Query heads per KV head of 1 and 4 (the other columns of the query operand are zero)."""
    p = Pair(cfg(n_q_heads=hq, tail_len=32, tail_slack=32, tail_dtype=2))
    k, v = small_tokens(60 + hq, 400, 2, 256)
    q = small_query(61 + hq, 400, hq, 256)
    got, want = run_prefill(p, 0, [1], [250], k[:250], v[:250], q[:250])
    assert max_err(got, want) <= TOL
    got, want = run_prefill(p, 0, [1], [150], k[250:], v[250:], q[250:])
    assert max_err(got, want) <= TOL


def test_prefill_softmax_scale_and_a_block_straddling_the_boundary():
    """A ring of 4 with chunks that leave the body boundary inside query blocks, and an explicit scale."""
    p = Pair(cfg(tail_len=4, tail_slack=28, tail_dtype=1, k_bits=4, v_bits=4, kvarn=1))
    k, v = small_tokens(70, 300, 2, 256)
    q = small_query(71, 300, 16, 256)
    off = 0
    for n in (37, 13, 90, 5):
        got = p.gpu.prefill_attn(0, [0], [n], dev(k[off:off + n]), dev(v[off:off + n]), dev(q[off:off + n]),
                                 softmax_scale=0.03).cpu().numpy()
        p.ora.append(0, [0], [n], k[off:off + n], v[off:off + n])
        want = oracle.prefill_reference(p.ora, 0, [0], [n], q[off:off + n], scale=0.03)
        assert max_err(got, want) <= TOL
        p.evict(0, [0])
        off += n


def test_prefill_of_one_token_equals_decode():
    """A chunk of one token: append then dense decode over the cache (same values within rounding)."""
    p = Pair(cfg(tail_len=64, tail_slack=32, tail_dtype=1))
    k, v = small_tokens(80, 200, 2, 256)
    p.append(0, [0], [199], k[:199], v[:199])
    q = small_query(81, 1, 16, 256)
    got = p.gpu.prefill_attn(0, [0], [1], dev(k[199:]), dev(v[199:]), dev(q)).cpu().numpy()
    dec = p.gpu.decode_attn(0, [0], dev(q)).cpu().numpy()
    assert float(np.max(np.abs(got - dec))) <= 1e-4


def test_prefill_errors_leave_the_cache_unchanged():
    import torch
    from quantized_decode_attention_append_amd import kvq
    p = Pair(cfg(layout=1))
    k, v = small_tokens(90, 20, 2, 256)
    q = small_query(91, 20, 16, 256)
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.prefill_attn(0, [0], [20], dev(k), dev(v), dev(q))
    assert e.value.status == kvq.KVQ_E_INVALID
    p = Pair(cfg(kvarn=1, tail_len=16, tail_slack=16, tail_dtype=1))
    p.append(0, [0], [100], *small_tokens(92, 100, 2, 256))
    need = p.gpu.prefill_workspace_bytes(1, 20, 120)
    assert need > 256
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    before = p.gpu.lengths(0, 0)
    with pytest.raises(kvq.KvqError) as e:
        p.gpu.prefill_attn(0, [0], [20], dev(k), dev(v), dev(q), workspace=ws)
    assert e.value.status == kvq.KVQ_E_SIZE
    assert p.gpu.lengths(0, 0) == before
    got, want = run_prefill(p, 0, [0], [20], k, v, q)
    assert max_err(got, want) <= TOL


def _workload_prefill(p, wl, layer, seq, check_chunks, n_rows=6):
    """Prefill one sequence of a workload in its 4096-token chunks through kvq_prefill_attn; for the chunks listed,
    compare sampled rows (the first, the last, and random ones) with the oracle."""
    n = wl.contexts[seq]
    rng = np.random.default_rng(1000 + seq)
    n_chunks = (n + W.CHUNK - 1) // W.CHUNK
    for c_i in range(n_chunks):
        s = c_i * W.CHUNK
        m = min(W.CHUNK, n - s)
        k, v = W.kv_tokens(wl.cfg, layer, seq, s, m)
        q = W.prefill_queries(wl.cfg, layer, seq, s, m)
        print(f"{wl.name} seq {seq} chunk {c_i}/{n_chunks}", flush=True)
        got = p.gpu.prefill_attn(layer, [seq], [m], dev(k), dev(v), dev(q)).cpu().numpy()
        p.ora.append(layer, [seq], [m], k, v)
        if c_i in check_chunks or c_i - n_chunks in check_chunks:
            rows = sorted({0, m - 1, *[int(x) for x in rng.integers(0, m, size=n_rows - 2)]})
            want = oracle.prefill_reference(p.ora, layer, [seq], [m], q, rows)
            err = max_err(got[rows], want)
            assert err <= TOL, f"{wl.name} chunk {c_i}: max abs error {err:.3e}"
        assert np.all(np.isfinite(got))


def test_prefill_at_the_64k_workload_size():
    """Layer 0 of the K6/V5 + bf16 tail workload prefilled to 65,536 positions in 4096-token chunks; sampled rows
    of the first, a middle and the last chunk against the oracle, and the slab byte-exact at the end."""
    wl = W.workload(2)
    p = Pair(dict(wl.cache_config(), n_layers=1))
    _workload_prefill(p, wl, 0, 0, check_chunks=(0, 7, -1))
    p.lengths_match(0, 0)
    p.assert_slab_equal(0, 0)


def test_prefill_kvarn_workload_sequence():
    """The KVarN K4/V4 + bf16 tail workload: its 16k-position stream, sampled rows of every chunk."""
    wl = W.workload(3)
    p = Pair(dict(wl.cache_config(), n_layers=1))
    seq = int(np.argmin(wl.contexts))
    _workload_prefill(p, wl, 0, seq, check_chunks=tuple(range(8)))
    p.lengths_match(0, seq)
    p.assert_slab_equal(0, seq)
