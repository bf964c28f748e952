"""GPU parity of token-axis K (KIVI-style: a K block is the 32 positions of one channel in a position tile, Qwen3.8-27B
page, reader comment on per-channel K) through the C ABI: slabs byte-exact with the oracle's packed image (codes and
per-channel scales, qN_0 or qN_1) while the body grows by whole tiles, and attention within 2e-3 of the oracle's
fp64 result for decode, the decode step, multi-query decode and chunked prefill."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import Pair, TOL, dev, max_err
from workloads import small_tokens, small_query

pytestmark = pytest.mark.gpu


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=3, capacity=1024, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=4,
             v_bits=4, kvarn=0, tail_len=64, tail_slack=64, tail_dtype=1, layout=0, k_axis=1)
    c.update(kw)
    return c


# (k_bits, v_bits, k_min, v_min, tail_len, tail_dtype, kvarn)
CASES = [
    (4, 4, 0, 0, 64, 1, 0),
    (2, 3, 0, 0, 1, 1, 0),     # the smallest window: the ring holds the tile still filling
    (6, 5, 0, 0, 64, 2, 0),    # K6/V5 with the 8-bit ring
    (4, 4, 0, 0, 32, 3, 1),    # f16 tail, KVarN
    (5, 5, 1, 1, 64, 1, 0),    # q5_1 token-axis K with a q5_1 V
    (8, 6, 1, 0, 96, 2, 1),
    (3, 8, 0, 0, 64, 1, 0),
]


def _ids(c):
    return f"K{c[0]}{'_1' if c[2] else '_0'}-V{c[1]}{'_1' if c[3] else '_0'}-W{c[4]}-t{c[5]}-kvarn{c[6]}"


def _pair(case, **kw):
    k, v, km, vm, w, t, kv = case
    slack = 64 + (32 - w % 32) % 32   # the ring (tail_len + tail_slack) is a whole number of tiles
    return Pair(cfg(k_bits=k, v_bits=v, k_min=km, v_min=vm, tail_len=w, tail_slack=slack, tail_dtype=t, kvarn=kv, **kw))


def _scales(seed):
    rng = np.random.default_rng(seed)
    return np.abs(rng.standard_t(3, size=(2, 2, 256))) + 0.05


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_token_axis_slabs_and_decode_match_oracle(case):
    p = _pair(case)
    seed = 5 * sum(case) + case[0]
    k, v = small_tokens(seed, 800, 2, 256, scale=_scales(seed))
    seqs = [0, 2]
    off = 0
    for n_new in ([150, 33], [1, 1], [1, 2], [210, 97], [1, 1], [40, 0]):
        n = sum(n_new)
        p.append(1, seqs, n_new, k[off:off + n], v[off:off + n])
        off += n
        p.evict(1, seqs)
        for s in seqs:
            p.lengths_match(1, s)
            assert p.gpu.lengths(1, s)[1] % 32 == 0
            p.assert_slab_equal(1, s)
        q = small_query(seed + off, 2, 16, 256)
        got, want = p.decode(1, seqs, q)
        assert max_err(got, want) <= TOL, (n_new, max_err(got, want))


@pytest.mark.parametrize("case", CASES[:5], ids=_ids)
def test_token_axis_decode_step_multi_query_and_prefill(case):
    p = _pair(case, capacity=2048)
    seed = 13 * sum(case)
    k, v = small_tokens(seed, 1400, 2, 256, scale=_scales(seed))
    q = small_query(seed + 2, 1400, 16, 256)
    seqs = [0, 1]
    off = 0
    for n_new in ([300, 120], [77, 200]):
        n = sum(n_new)
        got = p.gpu.prefill_attn(0, seqs, n_new, dev(k[off:off + n]), dev(v[off:off + n]),
                                 dev(q[off:off + n])).cpu().numpy()
        p.ora.append(0, seqs, n_new, k[off:off + n], v[off:off + n])
        want = oracle.prefill_reference(p.ora, 0, seqs, n_new, q[off:off + n])
        assert max_err(got, want) <= TOL, max_err(got, want)
        off += n
    for st in range(40):   # crosses a tile boundary of the body
        kk, vv, qq = k[off:off + 2], v[off:off + 2], q[off:off + 2]
        off += 2
        got = p.gpu.decode_step(0, seqs, dev(kk), dev(vv), dev(qq)).cpu().numpy()
        p.ora.append(0, seqs, [1, 1], kk, vv)
        p.ora.tail_evict(0, seqs)
        if st % 13 == 0 or st == 39:
            want = oracle.decode_reference(p.ora, 0, seqs, qq)
            assert max_err(got, want) <= TOL, (st, max_err(got, want))
            for s in seqs:
                p.lengths_match(0, s)
                p.assert_slab_equal(0, s)
    p.append(0, seqs, [8, 8], k[off:off + 16], v[off:off + 16])
    qm = small_query(seed + 9, 16, 16, 256).reshape(2, 8, 16, 256)
    got = p.gpu.decode_attn_multi(0, seqs, dev(qm).view(2, 8, 16, 256)).cpu().numpy()
    want = oracle.multi_query_reference(p.ora, 0, seqs, qm)
    assert max_err(got, want) <= TOL, max_err(got, want)


def test_token_axis_long_context():
    """K4/V4 token-axis K with a 2,048-position bf16 window at 12k positions: hundreds of K tiles per head."""
    p = Pair(cfg(n_layers=1, max_seqs=1, capacity=12288 + 64, tail_len=2048, tail_slack=512))
    k, v = small_tokens(91, 12288, 2, 256, scale=_scales(91))
    for s0 in range(0, 12288, 4096):
        p.append(0, [0], [4096], k[s0:s0 + 4096], v[s0:s0 + 4096])
    p.evict(0, [0])
    p.assert_slab_equal(0, 0)
    q = small_query(92, 1, 16, 256)
    got, want = p.decode(0, [0], q)
    assert max_err(got, want) <= TOL, max_err(got, want)
