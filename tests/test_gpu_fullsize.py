"""Parity at the workloads' full sizes (one layer each), in the launch configuration bench.py times.

At these sizes every work-group of the decode kernel covers many 32-position tiles, so the waves take further
tiles from the work-group counter, the online softmax rescales across tiles and the split merge combines
about a hundred partials per KV head: paths the small parity cases do not reach.  The oracle decodes the
whole context in fp64 (about a second per call at 65,536 positions)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import TOL, Pair, dev, max_err

pytestmark = pytest.mark.gpu


def prefill_all(p, wl, layer):
    for seq, n in enumerate(wl.contexts):
        for s in range(0, n, W.CHUNK):
            k, v = W.kv_tokens(wl.cfg, layer, seq, s, min(W.CHUNK, n - s))
            p.append(layer, [seq], [k.shape[0]], k, v)
    p.evict(layer, list(range(wl.batch)))


def step_inputs(wl, layer, st):
    """One decode step's appended token (all sequences, packed) and queries."""
    ks, vs = zip(*[W.decode_token(wl.cfg, layer, seq, st) for seq in range(wl.batch)])
    q = np.stack([W.query(wl.cfg, layer, seq, st) for seq in range(wl.batch)])
    return np.concatenate(ks), np.concatenate(vs), q


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_dense_decode_full_size(cfg_id):
    """Layer 0 of the workload at its full context (all sequences): cache bytes after the prefill, then decode
    steps as bench.py runs them (append 1 + evict + decode), each within the tolerance of the oracle and
    repeatable."""
    wl = W.workload(cfg_id)
    cfg = dict(wl.cache_config(), n_layers=1)
    p = Pair(cfg)
    prefill_all(p, wl, 0)
    seqs = list(range(wl.batch))
    for seq in seqs:
        p.lengths_match(0, seq)
    p.assert_slab_equal(0, wl.batch - 1)
    for st in range(max(1, min(2, wl.decode_steps))):
        k, v, q = step_inputs(wl, 0, st)
        if wl.decode_steps:   # the single-layer q8_0 workload decodes its prefill as is
            # as bench.py runs a step: append, evict and decode in one call
            got = p.gpu.decode_step(0, seqs, dev(k), dev(v), dev(q)).cpu().numpy()
            p.ora.append(0, seqs, [1] * wl.batch, k, v)
            p.ora.tail_evict(0, seqs)
            for seq in seqs:
                p.lengths_match(0, seq)
            p.assert_slab_equal(0, 0)
            want = oracle.decode_reference(p.ora, 0, seqs, q)
        else:
            got, want = p.decode(0, seqs, q)
        err = max_err(got, want)
        assert err <= TOL, f"{wl.name} step {st}: max abs error {err:.3e}"
        for _ in range(2):
            again = p.gpu.decode_attn(0, seqs, dev(q)).cpu().numpy()
            d = float(np.max(np.abs(again - got)))
            assert d <= 1e-5 * max(1.0, float(np.max(np.abs(got)))), f"{wl.name} step {st}: repeat differs by {d:.3e}"


def test_sparse_decode_full_size():
    """The sparse workload's layer 0: 262,144 positions, budgets of 2048 (512 newest + 1536 drawn) per step."""
    wl = W.workload(5)
    cfg = dict(wl.cache_config(), n_layers=1)
    p = Pair(cfg)
    prefill_all(p, wl, 0)
    n = wl.contexts[0]
    for st in range(2):
        k, v, q = step_inputs(wl, 0, st)
        p.append(0, [0], [1], k, v)
        pos = W.sparse_positions(wl.cfg, 0, 0, st, n + st + 1, wl.budget, wl.recent)[None]
        got, want = p.sparse(0, [0], q, pos)
        err = max_err(got, want)
        assert err <= TOL, f"{wl.name} step {st}: max abs error {err:.3e}"


def test_sparse_step_and_dense_rows_full_size():
    """The sparse workload's layer 0 as bench.py runs it: fused sparse steps (append inside the gather launch,
    the new position sometimes in the list), the slab byte-exact afterwards, then dense decode of the whole
    262,144-position row-layout cache (the gather kernel over every position) against the oracle."""
    import torch
    wl = W.workload(5)
    cfg = dict(wl.cache_config(), n_layers=1)
    p = Pair(cfg)
    prefill_all(p, wl, 0)
    n = wl.contexts[0]
    for st in range(2):
        k, v, q = step_inputs(wl, 0, st)
        pos = W.sparse_positions(wl.cfg, 0, 0, st, n + st + 1, wl.budget, wl.recent)[None]
        assert (pos == n + st).any()   # the newest positions are forced: the appended one is listed
        pos_d = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).to("cuda")
        got = p.gpu.sparse_decode_step(0, [0], dev(k), dev(v), dev(q), pos_d).cpu().numpy()
        p.ora.append(0, [0], [1], k, v)
        want = oracle.sparse_reference(p.ora, 0, [0], q, pos)
        err = max_err(got, want)
        assert err <= TOL, f"{wl.name} fused step {st}: max abs error {err:.3e}"
    p.lengths_match(0, 0)
    p.assert_slab_equal(0, 0)
    q = W.query(wl.cfg, 0, 0, 7)[None]
    got, want = p.decode(0, [0], q)
    err = max_err(got, want)
    assert err <= TOL, f"{wl.name} dense decode of the row layout: max abs error {err:.3e}"
