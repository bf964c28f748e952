"""The decode-step calls captured into a HIP graph (torch.cuda.CUDAGraph on the caller's stream) and replayed.

Capture runs no kernel but advances the cache's host state by the captured step, so a replay performs that
step: its append writes the same ring or body row again and its decode reads the same rows, and every replay
must give the oracle's bytes and outputs. Eager calls run between the replays (they share the stream and the
workspace), and each replay is checked on its own.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import Pair, TOL, dev, max_err
from workloads import small_tokens, small_query

pytestmark = pytest.mark.gpu


def cfg(**kw):
    c = dict(n_layers=2, max_seqs=2, capacity=1024, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=6,
             v_bits=5, kvarn=0, tail_len=0, tail_slack=0, tail_dtype=0)
    c.update(kw)
    return c


def capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    return g


@pytest.mark.parametrize("tail_dtype,kvarn", [(1, 0), (2, 1), (3, 0)])
def test_decode_step_graph(tail_dtype, kvarn):
    import torch
    p = Pair(cfg(tail_len=64, tail_slack=32, tail_dtype=tail_dtype, kvarn=kvarn))
    k, v = small_tokens(300 + tail_dtype, 400, 2, 256)
    seqs = [0, 1]
    p.append(1, [0], [200], k[:200], v[:200])
    p.append(1, [1], [70], k[200:270], v[200:270])
    p.evict(1, seqs)
    kk, vv, q = dev(k[270:272]), dev(v[270:272]), dev(small_query(301, 2, 16, 256))
    out = torch.zeros((2, 16, 256), dtype=torch.float32, device="cuda")
    ws = p.gpu.workspace(2, 400)
    g = capture(torch, lambda: p.gpu.decode_step(1, seqs, kk, vv, q, out=out, workspace=ws))
    p.ora.append(1, seqs, [1, 1], k[270:272], v[270:272])
    p.ora.tail_evict(1, seqs)
    want = oracle.decode_reference(p.ora, 1, seqs, small_query(301, 2, 16, 256))
    q2 = small_query(302, 2, 16, 256)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert max_err(got, want) <= TOL, f"replay {rep}: {max_err(got, want):.3e}"
        for i in seqs:
            p.lengths_match(1, i)
            p.assert_slab_equal(1, i)
        # eager work on the same stream and workspace between the replays
        e_got = p.gpu.decode_attn(1, seqs, dev(q2), workspace=ws).cpu().numpy()
        assert max_err(e_got, oracle.decode_reference(p.ora, 1, seqs, q2)) <= TOL


@pytest.mark.parametrize("fused", [False, True])
def test_sparse_step_graph(fused):
    """Append + sparse decode, as two calls or as kvq_sparse_decode_step (the append inside the gather launch)."""
    import torch
    p = Pair(cfg(k_bits=8, v_bits=8, layout=1))
    k, v = small_tokens(310, 600, 2, 256)
    p.append(0, [0], [500], k[:500], v[:500])
    rng = np.random.default_rng(311)
    pos = np.concatenate([np.arange(501 - 64, 501), rng.choice(501 - 64, size=192, replace=False)]).astype(np.int32)
    q = small_query(312, 1, 16, 256)
    kk, vv, qd = dev(k[500:501]), dev(v[500:501]), dev(q)
    posd = torch.from_numpy(pos[None].copy()).to("cuda")
    out = torch.zeros((1, 16, 256), dtype=torch.float32, device="cuda")
    ws = p.gpu.workspace(1, 256)

    def step():
        if fused:
            p.gpu.sparse_decode_step(0, [0], kk, vv, qd, posd, out=out, workspace=ws)
        else:
            p.gpu.append(0, [0], [1], kk, vv)
            p.gpu.sparse_decode_attn(0, [0], qd, posd, out=out, workspace=ws)

    g = capture(torch, step)
    p.ora.append(0, [0], [1], k[500:501], v[500:501])
    want = oracle.sparse_reference(p.ora, 0, [0], q, pos[None])
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert max_err(got, want) <= TOL, f"replay {rep}: {max_err(got, want):.3e}"
        p.lengths_match(0, 0)
        p.assert_slab_equal(0, 0)
        e_got, e_want = p.sparse(0, [0], small_query(313 + rep, 1, 16, 256), pos[None])
        assert max_err(e_got, e_want) <= TOL


@pytest.mark.parametrize("layout", [0, 1])
def test_multi_query_graph(layout):
    """kvq_decode_attn_multi captured and replayed (8 queries on each of two sequences), eager single-query
    decode on the same stream and workspace between the replays; every replay matches the eager call bit for bit
    and the oracle within the tolerance."""
    import torch
    p = Pair(cfg(tail_len=64, tail_slack=32, tail_dtype=1, layout=layout))
    k, v = small_tokens(320 + layout, 500, 2, 256)
    seqs = [0, 1]
    p.append(0, seqs, [260, 90], k[:350], v[:350])
    p.evict(0, seqs)
    p.append(0, seqs, [8, 8], k[350:366], v[350:366])
    qn = small_query(321, 16, 16, 256).reshape(2, 8, 16, 256)
    q = dev(qn).view(2, 8, 16, 256)
    out = torch.zeros((2, 8, 16, 256), dtype=torch.float32, device="cuda")
    ws = p.gpu.workspace(16, 400)
    eager = p.gpu.decode_attn_multi(0, seqs, q, out=torch.empty_like(out), workspace=ws).cpu().numpy()
    want = oracle.multi_query_reference(p.ora, 0, seqs, qn)
    assert max_err(eager, want) <= TOL
    g = capture(torch, lambda: p.gpu.decode_attn_multi(0, seqs, q, out=out, workspace=ws))
    q1 = small_query(322, 2, 16, 256)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), eager, err_msg=f"replay {rep}")
        e_got = p.gpu.decode_attn(0, seqs, dev(q1), workspace=ws).cpu().numpy()
        assert max_err(e_got, oracle.decode_reference(p.ora, 0, seqs, q1)) <= TOL
