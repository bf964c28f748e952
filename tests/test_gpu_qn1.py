"""GPU parity of qN_1 bodies (a scale and a minimum per 32 values: the BeeLlama page's q2_1 .. q6_1 and the KVarN
benchmark page's q5_1 and q8_0-q5_1) through the C ABI: slabs byte-exact with the oracle's packed image after
appends and evictions (codes, scales and minima), and attention within 2e-3 of the oracle's fp64 result for
single-query decode, the decode step, multi-query decode and chunked prefill."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import Pair, TOL, dev, max_err
from workloads import small_tokens, small_query

pytestmark = pytest.mark.gpu


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=3, capacity=1024, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=5,
             v_bits=5, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0, layout=0, k_min=1, v_min=1)
    c.update(kw)
    return c


# (k_bits, v_bits, k_min, v_min, tail_dtype, kvarn): the pages' pairs and every width on one side or the other
CASES = [
    (5, 5, 1, 1, 0, 0),   # q5_1
    (8, 5, 0, 1, 0, 0),   # q8_0-q5_1
    (2, 2, 1, 1, 1, 0),   # q2_1 with a bf16 tail
    (3, 3, 1, 1, 2, 0),   # q3_1 with the 8-bit ring
    (6, 6, 1, 1, 3, 1),   # q6_1, f16 tail, KVarN
    (4, 7, 1, 0, 1, 1),   # q4_1-q7_0, KVarN
    (8, 8, 1, 1, 0, 0),   # q8_1
    (6, 5, 0, 1, 2, 0),   # K6/V5 with a qN_1 V and the 8-bit ring
    (7, 4, 1, 0, 0, 0),
]


def _ids(c):
    k, v, km, vm, t, kv = c
    return f"K{k}{'_1' if km else '_0'}-V{v}{'_1' if vm else '_0'}-t{t}-kvarn{kv}"


def _pair(case, **kw):
    k, v, km, vm, t, kv = case
    tail = dict(tail_len=64, tail_slack=32, tail_dtype=t) if t else {}
    return Pair(cfg(k_bits=k, v_bits=v, k_min=km, v_min=vm, kvarn=kv, **tail, **kw))


def _scales(seed):
    """Per-(head, K/V, channel) scales and an offset pattern, so blocks are far from zero-centred."""
    rng = np.random.default_rng(seed)
    return np.abs(rng.standard_t(3, size=(2, 2, 256))) + 0.05


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_qn1_slabs_and_decode_match_oracle(case):
    p = _pair(case)
    seed = 3 * sum(case) + case[0]
    k, v = small_tokens(seed, 700, 2, 256, scale=_scales(seed))
    # shift K and V by a per-channel offset (what a minimum is for)
    off = np.random.default_rng(seed + 1).normal(0, 2, size=(2, 256)).astype(np.float32)
    from workloads import bf16_bits, bf16_to_f32
    k = bf16_bits(bf16_to_f32(k) + off)
    v = bf16_bits(bf16_to_f32(v) - 0.5 * off)
    seqs = [0, 2]
    off_t = 0
    for n_new in ([150, 33], [1, 1], [210, 97], [1, 1]):
        n = sum(n_new)
        p.append(1, seqs, n_new, k[off_t:off_t + n], v[off_t:off_t + n])
        off_t += n
        p.evict(1, seqs)
        for s in seqs:
            p.lengths_match(1, s)
            p.assert_slab_equal(1, s)
        q = small_query(seed + off_t, 2, 16, 256)
        got, want = p.decode(1, seqs, q)
        assert max_err(got, want) <= TOL, (n_new, max_err(got, want))


@pytest.mark.parametrize("case", CASES[:5], ids=_ids)
def test_qn1_decode_step_multi_query_and_prefill(case):
    p = _pair(case, capacity=2048)
    seed = 11 * sum(case)
    k, v = small_tokens(seed, 1400, 2, 256, scale=_scales(seed))
    q = small_query(seed + 2, 1400, 16, 256)
    seqs = [0, 1]
    # chunked prefill (append + attention of the chunk's queries)
    off_t = 0
    for n_new in ([300, 120], [77, 200]):
        n = sum(n_new)
        got = p.gpu.prefill_attn(0, seqs, n_new, dev(k[off_t:off_t + n]), dev(v[off_t:off_t + n]),
                                 dev(q[off_t:off_t + n])).cpu().numpy()
        p.ora.append(0, seqs, n_new, k[off_t:off_t + n], v[off_t:off_t + n])
        want = oracle.prefill_reference(p.ora, 0, seqs, n_new, q[off_t:off_t + n])
        assert max_err(got, want) <= TOL, max_err(got, want)
        off_t += n
    # decode steps (append 1 + evict + attention, in separate launches for a qN_1 body)
    for st in range(3):
        kk, vv = k[off_t:off_t + 2], v[off_t:off_t + 2]
        qq = q[off_t:off_t + 2]
        off_t += 2
        got = p.gpu.decode_step(0, seqs, dev(kk), dev(vv), dev(qq)).cpu().numpy()
        p.ora.append(0, seqs, [1, 1], kk, vv)
        p.ora.tail_evict(0, seqs)
        want = oracle.decode_reference(p.ora, 0, seqs, qq)
        assert max_err(got, want) <= TOL, (st, max_err(got, want))
        for s in seqs:
            p.lengths_match(0, s)
            p.assert_slab_equal(0, s)
    # multi-query decode of 8 drafts
    p.append(0, seqs, [8, 8], k[off_t:off_t + 16], v[off_t:off_t + 16])
    qm = small_query(seed + 9, 16, 16, 256).reshape(2, 8, 16, 256)
    got = p.gpu.decode_attn_multi(0, seqs, dev(qm).view(2, 8, 16, 256)).cpu().numpy()
    want = oracle.multi_query_reference(p.ora, 0, seqs, qm)
    assert max_err(got, want) <= TOL, max_err(got, want)


def test_qn1_long_context_and_noalloc():
    """q8_0-q5_1 at 16k positions (one sequence, bf16 tail 1024): several hundred tiles per KV head across the
    splits; kvq_decode_attn_noalloc gives the same result."""
    p = Pair(cfg(n_layers=1, max_seqs=1, capacity=16384 + 64, k_bits=8, v_bits=5, k_min=0, v_min=1, tail_len=1024,
                 tail_slack=512, tail_dtype=1))
    k, v = small_tokens(77, 16384, 2, 256, scale=_scales(77))
    for s0 in range(0, 16384, 4096):
        p.append(0, [0], [4096], k[s0:s0 + 4096], v[s0:s0 + 4096])
    p.evict(0, [0])
    p.assert_slab_equal(0, 0)
    q = small_query(78, 1, 16, 256)
    got, want = p.decode(0, [0], q)
    assert max_err(got, want) <= TOL, max_err(got, want)
    import torch
    out = torch.empty((1, 16, 256), dtype=torch.float32, device="cuda")
    p.gpu.decode_attn_noalloc(0, [0], dev(q), out)
    assert float(np.max(np.abs(out.cpu().numpy() - got))) <= 1e-5


def test_qn1_refused_on_the_row_layout():
    from quantized_decode_attention_append_amd import kvq
    with pytest.raises(kvq.KvqError) as e:
        kvq.Cache(cfg(layout=1))
    assert e.value.status == kvq.KVQ_E_INVALID
