"""Pins of the algorithmic byte counts behind every GB/s figure: the oracle's ``sizes`` module and bench.py's own
copies (the numerator of the JSON line's ``value`` and ``roofline.achieved``).

Expected values are derived here from what the pages print, not from either implementation:

* row bytes of one token x one KV head x (K or V) from the BeeLlama page's KV MiB column (16 layers x 4 KV heads
  x 65,536 positions, tail 0): q8_0 2176 MiB, q6_0 1664, q5_0 1408, q4_0 1152;
* the bf16 row of 2 KV heads x 256 x (K, V) x 2 bytes = 2,048 bytes per token per layer, and its 2,048-position
  budget of 4 MiB per layer, from the offload page's byte arithmetic (``tests/golden/p2_qsa_bytes.csv``).

From those, the per-call KV figures of the five synthetic workloads are 4,456,448 B (q8_0, 4,096 positions),
(len - 2048) * 768 + 2048 * 2048 (K6/V5 + bf16 tail), the sum over streams of (len - 1024) * 576 + 1024 * 2048
plus 2 KiB of KVarN scales each (KVarN K4/V4 + bf16 tail), 201,981,952 B (K6/V5 + q8_0 ring at 262,144) and
2,228,224 B (q8_0 budget of 2,048). A call also reads its bf16 query rows and writes its fp32 output rows:
16 heads x 256 x (2 + 4) = 24,576 bytes per query vector.
"""
import csv
import os

import numpy as np
import pytest

import bench
import oracle
import workloads as W
from oracle import sizes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _csv(name):
    with open(os.path.join(GOLD, name)) as f:
        return list(csv.DictReader(line for line in f if not line.startswith("#")))


def _table_row_bytes():
    """Row bytes per (token, KV head, K or V) of q4_0..q8_0 from the KV MiB table at tail 0."""
    bits = {"q4_0": 4, "q5_0": 5, "q6_0": 6, "q8_0": 8}
    out = {}
    for r in _csv("p5_kv_mib.csv"):
        if int(r["tail"]) == 0:
            total = int(float(r["kv_mib"]) * 2 ** 20)
            assert total % (16 * 65536 * 4 * 2) == 0
            out[bits[r["cache"]]] = total // (16 * 65536 * 4 * 2)
    return out


ROW = _table_row_bytes()
P2 = {r["quantity"]: int(r["bytes"]) for r in _csv("p2_qsa_bytes.csv")}
BF16_TOKEN = P2["bf16_row_per_token_per_layer"]          # 2 KV heads, K and V
QO = 16 * 256 * (2 + 4)                                    # bf16 query read + fp32 output written per query vector


def test_table_row_bytes():
    assert ROW == {4: 144, 5: 176, 6: 208, 8: 272}
    assert BF16_TOKEN == 2048


def test_ring_token_bytes_every_dtype():
    # bf16 and f16 rings hold 16-bit values: the page's unquantized row; the q8_0 ring holds q8_0 rows
    assert sizes.ring_token_bytes(1, 2, 256) == BF16_TOKEN
    assert sizes.ring_token_bytes(3, 2, 256) == BF16_TOKEN
    assert sizes.ring_token_bytes(2, 2, 256) == 2 * 2 * ROW[8] == 1088
    assert sizes.ring_token_bytes(0, 2, 256) == 0


def _expected_kv(wid, lens, bodies):
    """Per-call KV bytes of workload wid from the table's row sizes (2 KV heads)."""
    if wid == 1:
        return sum(n * 2 * 2 * ROW[8] for n in lens)
    if wid in (2, 4):
        body = 2 * (ROW[6] + ROW[5])
        ring = BF16_TOKEN if wid == 2 else 2 * 2 * ROW[8]
        return sum(b * body + (n - b) * ring for n, b in zip(lens, bodies))
    if wid == 3:
        return sum(b * 2 * 2 * ROW[4] + (n - b) * BF16_TOKEN + 2 * 2 * 256 * 2 for n, b in zip(lens, bodies))
    raise ValueError(wid)


def test_workload_figures():
    # the workloads' first timed call, in the lengths the cache holds at that call
    assert _expected_kv(1, [4096], [4096]) == 4_456_448
    assert _expected_kv(4, [262144], [262144 - 2048]) == 201_981_952
    assert _expected_kv(2, [65537], [65537 - 2048]) == (65537 - 2048) * 768 + 2048 * 2048
    assert 2048 * 2 * 2 * ROW[8] == 2_228_224 == P2["budget_2048_per_layer"] * 34 // 64


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_dense_call_bytes_pinned(wid):
    wl = W.workload(wid)
    cfg = wl.cache_config()
    lens = [n + (1 if wl.decode_steps else 0) for n in wl.contexts]
    bodies = [max(0, n - wl.tail_len) if wl.tail_len else n for n in lens]
    kv = _expected_kv(wid, lens, bodies)
    n = len(lens)
    assert bench.decode_kv_bytes(cfg, lens, bodies) == kv
    assert bench.decode_call_bytes(cfg, lens, bodies) == kv + n * QO
    assert sizes.decode_kv_bytes(cfg, lens, bodies) == kv
    assert sizes.decode_bytes(cfg, lens, bodies) == kv + n * QO
    if wid == 4:
        assert bench.decode_call_bytes(cfg, lens, bodies) == 201_981_952 + QO
    if wid == 1:
        assert bench.decode_call_bytes(cfg, lens, bodies) == 4_456_448 + QO


def test_sparse_call_bytes_pinned():
    wl = W.workload(5)
    cfg = wl.cache_config()
    assert bench.sparse_kv_bytes(cfg, wl.budget, 1) == 2_228_224
    assert bench.sparse_call_bytes(cfg, wl.budget, 1) == 2_228_224 + QO
    assert sizes.sparse_kv_bytes(cfg, wl.budget, 0) == 2_228_224
    # the offload page's bf16-equivalent budget read, scaled by q8_0's 34 bytes per 64
    assert bench.sparse_kv_bytes(cfg, wl.budget, 1) * 64 == P2["budget_2048_per_layer"] * 34


def test_oracle_bytes_follow_the_cache_state():
    """decode_bytes over the lengths an oracle cache reports after appends and evicts (every ring kind, KVarN)
    equals the row count times the table's row sizes."""
    rng = np.random.default_rng(5)
    for tail_dtype, kvarn, kb, vb in ((1, 0, 6, 5), (2, 0, 6, 5), (3, 1, 4, 4), (0, 0, 8, 8), (2, 1, 5, 4)):
        cfg = dict(n_layers=1, max_seqs=2, capacity=512, n_q_heads=16, n_kv_heads=2, head_dim=256, k_bits=kb,
                   v_bits=vb, kvarn=kvarn, tail_len=64 if tail_dtype else 0, tail_slack=32 if tail_dtype else 0,
                   tail_dtype=tail_dtype)
        o = oracle.OracleCache(cfg)
        n = [int(x) for x in rng.integers(70, 300, size=2)]
        k, v = W.small_tokens(3, sum(n), 2, 256)
        o.append(0, [0, 1], n, k, v)
        o.tail_evict(0, [0, 1])
        lens = [o.lengths(0, s) for s in (0, 1)]
        ring_tok = {0: 0, 1: BF16_TOKEN, 2: 1088, 3: BF16_TOKEN}[tail_dtype]
        body_tok = 2 * (ROW.get(kb, 0) + ROW.get(vb, 0)) if kb in ROW and vb in ROW else None
        want = sum(b * body_tok + (ln - b) * ring_tok + (2048 if kvarn else 0) for ln, b in lens)
        got = sizes.decode_kv_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens])
        assert got == want
        assert bench.decode_kv_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens]) == want
        assert sizes.decode_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens]) == want + 2 * QO
