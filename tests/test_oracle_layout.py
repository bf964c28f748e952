"""Pins of the oracle's arena size and byte layout.

Sizes are pinned to the values the pages print (``tests/golden``): the KV MiB table
of the BeeLlama.cpp v0.4.1 page, the cache-size column of the KVarN benchmark page,
the QSA byte arithmetic of the offload page and the memory delta of the Qwen3.8-27B
page. The bit layout is a design choice; it is pinned by hand-worked byte examples
of the rule stated in the format description and by pack/unpack round trips.
"""
import csv
import os

import numpy as np
import pytest

from oracle import layout, sizes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _csv(name):
    with open(os.path.join(GOLD, name)) as f:
        return list(csv.DictReader(line for line in f if not line.startswith("#")))


BITS = {"q4_0": 4, "q5_0": 5, "q6_0": 6, "q8_0": 8}
TYPES = {**{k: (v, False) for k, v in BITS.items()}, "q5_1": (5, True)}   # (bits, scale + minimum)


def _cfg(**kw):
    c = dict(n_layers=16, max_seqs=1, capacity=65536, n_q_heads=32, n_kv_heads=4, head_dim=256,
             k_bits=4, v_bits=4, kvarn=0, tail_len=0, tail_slack=512, tail_dtype=1)
    c.update(kw)
    return c


@pytest.mark.parametrize("row", _csv("p5_kv_mib.csv"), ids=lambda r: f"{r['cache']}-t{r['tail']}")
def test_kv_mib_table_exact(row):
    n = BITS[row["cache"]]
    cfg = _cfg(k_bits=n, v_bits=n, tail_len=int(row["tail"]))
    assert layout.cache_bytes(cfg) == int(float(row["kv_mib"]) * 2 ** 20)


@pytest.mark.parametrize("row", _csv("p3_cache_size.csv"), ids=lambda r: f"{r['k_type']}-{r['v_type']}")
def test_cache_size_percent_of_bf16(row):
    (k, kmin), (v, vmin) = TYPES[row["k_type"]], TYPES[row["v_type"]]
    q = sizes.kv_token_bytes(k, v, 4, 256, kmin, vmin)
    bf = sizes.bf16_token_bytes(4, 256)
    assert round(100.0 * q / bf, 1) == float(row["percent"])
    # and the whole cache at the table's shape keeps the same ratio exactly
    cfg = _cfg(k_bits=k, v_bits=v, k_min=int(kmin), v_min=int(vmin))
    assert layout.cache_bytes(cfg) * bf == q * 16 * 65536 * bf


def test_qsa_bf16_byte_arithmetic():
    g = {r["quantity"]: int(r["bytes"]) for r in _csv("p2_qsa_bytes.csv")}
    per_tok = sizes.bf16_token_bytes(2, 256)
    assert per_tok == g["bf16_row_per_token_per_layer"]
    assert per_tok * 262144 == g["layer_at_262144_tokens"]
    assert per_tok * 262144 * 12 == g["all_12_layers_per_step"]
    assert per_tok * 2048 == g["budget_2048_per_layer"]
    assert per_tok * 2048 * 12 == g["budget_2048_all_12_layers"]
    # a bf16 tail ring holding every position costs exactly the unquantized row
    assert sizes.ring_token_bytes(1, 2, 256) == per_tok
    # the q8_0 sparse read is the bf16-equivalent figure scaled by 34/64
    cfg = dict(n_kv_heads=2, head_dim=256, k_bits=8, v_bits=8, tail_dtype=0)
    assert sizes.sparse_bytes(cfg, 2048, 0) * 64 == g["budget_2048_per_layer"] * 34


def test_memory_delta_at_120k_is_about_1_1_gb():
    g = {r["quantity"]: float(r["value"]) for r in _csv("p4_memory_delta.csv")}
    ctx = int(g["context"])
    # shape read from the KV MiB table's model: 16 attention layers, 4 KV heads x 256
    q8 = _cfg(capacity=ctx, k_bits=8, v_bits=8)
    d = _cfg(capacity=ctx, k_bits=6, v_bits=5, tail_len=2048, tail_dtype=2)
    delta_gb = (layout.cache_bytes(q8) - layout.cache_bytes(d)) / 1e9
    page_delta = g["q8_0_gb"] - g["setting_d_gb"]
    assert abs(delta_gb - page_delta) <= 0.1 + 1e-9


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_row_and_tile_sizes(n_bits):
    for d in (128, 256):
        assert layout.row_bytes(n_bits, d) == d // 32 * (4 * n_bits + 2)
        u = np.zeros((1, 32, d), dtype=np.uint8)
        s = np.zeros((1, 32, d // 32), dtype=np.float16)
        assert layout.pack_v_tiles(u, s, n_bits).shape == (1, 32 * layout.row_bytes(n_bits, d))
        assert layout.pack_k_rows(u[0], s[0], n_bits).shape == (32, layout.row_bytes(n_bits, d))
        assert layout.pack_k_tiles(u, s, n_bits).shape == (1, 32 * layout.row_bytes(n_bits, d))


def test_piece_bits_worked_examples():
    # w = 4: e_i = i + 1; element i at bit 16*(i%2) + 4*(i//2)
    b = layout.pack_pieces(np.array([[1, 2, 3, 4, 5, 6, 7, 8]]), 4)
    assert list(b) == [0x31, 0x75, 0x42, 0x86]
    # w = 2: two pieces share a word; element i of piece p at 16*(i%2) + 8p + 2*(i//2)
    b = layout.pack_pieces(np.array([[0, 1, 2, 3, 0, 1, 2, 3], [3, 2, 1, 0, 3, 2, 1, 0]]), 2)
    assert list(b) == [0x88, 0x77, 0xDD, 0x22]
    # w = 1: four pieces share a word; element i of piece p at 16*(i%2) + 4p + i//2
    b = layout.pack_pieces(np.array([[(i + p) % 2 for i in range(8)] for p in range(4)]), 1)
    assert list(b) == [0xF0, 0xF0, 0x0F, 0x0F]
    # w = 8: e_i in byte i
    b = layout.pack_pieces(np.array([[9, 8, 7, 6, 5, 4, 3, 2]]), 8)
    assert list(b) == [9, 8, 7, 6, 5, 4, 3, 2]


def test_k_row_worked_example():
    # D = 256, N = 6: plane widths 4 then 2. One code set at channel 32*b + 8*j + i.
    d, n = 256, 6
    for (b, j, i, val) in [(0, 0, 0, 0x3F), (5, 2, 3, 0x2A), (7, 3, 7, 0x11), (2, 1, 6, 0x30)]:
        u = np.zeros((1, d), dtype=np.uint8)
        u[0, 32 * b + 8 * j + i] = val
        row = layout.pack_k_rows(u, np.zeros((1, 8), dtype=np.float16), n)[0]
        expect = np.zeros(layout.row_bytes(n, d), dtype=np.uint8)
        # nibble plane: [j][b] pieces of 4 bytes
        w0 = (val & 0xF) << (16 * (i % 2) + 4 * (i // 2))
        base = j * 32 + b * 4
        expect[base:base + 4] |= np.frombuffer(np.uint32(w0).tobytes(), dtype=np.uint8)
        # 2-bit plane after 128 bytes: [j][b-pair] words, piece p = b % 2
        w1 = (val >> 4) << (16 * (i % 2) + 8 * (b % 2) + 2 * (i // 2))
        base = 128 + j * 16 + (b // 2) * 4
        expect[base:base + 4] |= np.frombuffer(np.uint32(w1).tobytes(), dtype=np.uint8)
        assert np.array_equal(row, expect)


def test_v_tile_worked_example():
    # D = 256, N = 5: nibble plane (64 B per lane, 16-byte chunks), then 1-bit plane
    d, n = 256, 5
    for (t, ch, val) in [(0, 0, 0x1F), (5, 17, 0x13), (21, 255, 0x0A), (31, 128, 0x10)]:
        u = np.zeros((1, 32, d), dtype=np.uint8)
        u[0, t, ch] = val
        tile = layout.pack_v_tiles(u, np.zeros((1, 32, 8), dtype=np.float16), n)[0]
        expect = np.zeros(32 * layout.row_bytes(n, d), dtype=np.uint8)
        j = (t % 16) // 4
        i = t % 4 + 4 * (t // 16)
        lane = 16 * j + ch % 16
        nt = ch // 16
        # nibble plane: lane bytes 4*nt, interleaved in 16-byte chunks across 64 lanes
        lb = 4 * nt
        off = (lb // 16) * 1024 + lane * 16 + lb % 16
        w0 = (val & 0xF) << (16 * (i % 2) + 4 * (i // 2))
        expect[off:off + 4] |= np.frombuffer(np.uint32(w0).tobytes(), dtype=np.uint8)
        # 1-bit plane after 4096 bytes: 16 bytes per lane (one chunk); 4 pieces per word
        off = 4096 + lane * 16 + (nt // 4) * 4
        w1 = (val >> 4) << (16 * (i % 2) + 4 * (nt % 4) + i // 2)
        expect[off:off + 4] |= np.frombuffer(np.uint32(w1).tobytes(), dtype=np.uint8)
        assert np.array_equal(tile, expect)


def test_k_tile_worked_example():
    # D = 256, N = 5: nibble plane (32 B per lane run, two 16-byte chunks), then 1-bit plane (8 B per lane)
    d, n = 256, 5
    for (t, b, j, i, val, sc) in [(0, 0, 0, 0, 0x1F, 1.5), (17, 5, 2, 3, 0x13, -2.0), (31, 7, 3, 7, 0x0A, 0.25),
                                  (14, 2, 1, 6, 0x10, 3.0)]:
        u = np.zeros((1, 32, d), dtype=np.uint8)
        u[0, t, 32 * b + 8 * j + i] = val
        d16 = np.zeros((1, 32, 8), dtype=np.float16)
        d16[0, t, b] = sc
        tile = layout.pack_k_tiles(u, d16, n)[0]
        expect = np.zeros(32 * layout.row_bytes(n, d), dtype=np.uint8)
        s, m = t // 16, t % 16
        lane = 16 * j + m
        # subtile s starts at 512 * N * s; nibble plane: lane run byte 4b, 16-byte chunks over 64 lanes
        rb = 4 * b
        off = 512 * n * s + (rb // 16) * 1024 + lane * 16 + rb % 16
        w0 = (val & 0xF) << (16 * (i % 2) + 4 * (i // 2))
        expect[off:off + 4] |= np.frombuffer(np.uint32(w0).tobytes(), dtype=np.uint8)
        # 1-bit plane after 512 * 4 bytes of the subtile: 8 bytes per lane, 4 pieces per word
        off = 512 * n * s + 2048 + lane * 8 + (b // 4) * 4
        w1 = (val >> 4) << (16 * (i % 2) + 4 * (b % 4) + i // 2)
        expect[off:off + 4] |= np.frombuffer(np.uint32(w1).tobytes(), dtype=np.uint8)
        # scales [block][position] after the codes
        off = 1024 * n + 2 * (32 * b + t)
        expect[off:off + 2] = np.frombuffer(np.float16(sc).tobytes(), dtype=np.uint8)
        assert np.array_equal(tile, expect), (t, b, j, i)


def test_bf16_k_tile_worked_example():
    bits = np.zeros((1, 32, 256), dtype=np.uint16)
    bits[0, 19, 32 * 6 + 8 * 2 + 5] = 0xBEEF
    tile = layout.pack_bf16_k_tiles(bits)[0].view(np.uint16)
    # [s][b][lane][8]: s = 1, b = 6, lane = 16 * 2 + 3, element 5
    idx = ((1 * 8 + 6) * 64 + (16 * 2 + 3)) * 8 + 5
    assert tile[idx] == 0xBEEF and np.count_nonzero(tile) == 1


@pytest.mark.parametrize("n_bits", range(2, 9))
def test_pack_unpack_round_trip(n_bits):
    rng = np.random.default_rng(n_bits)
    for d in (128, 256):
        u = rng.integers(0, 1 << n_bits, size=(7, d)).astype(np.uint8)
        s = rng.standard_normal((7, d // 32)).astype(np.float16)
        u2, s2 = layout.unpack_k_rows(layout.pack_k_rows(u, s, n_bits), n_bits, d)
        assert np.array_equal(u, u2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))
        u = rng.integers(0, 1 << n_bits, size=(3, 32, d)).astype(np.uint8)
        s = rng.standard_normal((3, 32, d // 32)).astype(np.float16)
        u2, s2 = layout.unpack_v_tiles(layout.pack_v_tiles(u, s, n_bits), n_bits, d)
        assert np.array_equal(u, u2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))
        u2, s2 = layout.unpack_k_tiles(layout.pack_k_tiles(u, s, n_bits), n_bits, d)
        assert np.array_equal(u, u2) and np.array_equal(s.view(np.uint16), s2.view(np.uint16))
    b = rng.integers(0, 1 << 16, size=(2, 32, 256)).astype(np.uint16)
    assert np.array_equal(layout.unpack_bf16_v_tiles(layout.pack_bf16_v_tiles(b), 256), b)
    assert np.array_equal(layout.unpack_bf16_k_tiles(layout.pack_bf16_k_tiles(b), 256), b)


def test_slab_regions_are_disjoint_and_aligned():
    for kw in (dict(), dict(tail_len=2048), dict(tail_len=1024, tail_dtype=2, kvarn=1, k_bits=6, v_bits=5)):
        lay = layout.slab_layout(_cfg(**kw))
        spans = sorted(v for k, v in lay.items() if k in ("k_body", "v_body", "k_ring", "v_ring", "sigma"))
        end = 0
        for off, size in spans:
            assert off % 256 == 0 and off >= end
            end = off + size
        assert lay["slab"] >= end and lay["slab"] % 256 == 0


def test_qn1_rows_and_tiles_carry_the_minima_after_the_scales():
    """Hand-worked placement: a qN_1 K row ends with the 8 scales then the 8 minima (block order); a K tile
    ends with the scales [block][position] then the minima [position][block]; a V tile with the scales and then
    the minima, both [block][position]."""
    rng = np.random.default_rng(3)
    n = 5
    u = rng.integers(0, 32, size=(1, 32, 256)).astype(np.uint8)
    d = (np.arange(32 * 8).reshape(1, 32, 8) + 1).astype(np.float16)
    m = (-np.arange(32 * 8).reshape(1, 32, 8) - 0.5).astype(np.float16)
    rb0 = layout.row_bytes(n, 256)
    assert layout.row_bytes(n, 256, True) == rb0 + 16 == 8 * (4 * n + 4)
    rows = layout.pack_k_rows(u[0], d[0], n, m[0])
    assert rows.shape == (32, rb0 + 16)
    assert np.array_equal(rows[:, :rb0], layout.pack_k_rows(u[0], d[0], n))
    assert np.array_equal(rows[:, rb0:].copy().view(np.float16), m[0])
    kt = layout.pack_k_tiles(u, d, n, m)
    tb0 = 32 * rb0
    assert kt.shape == (1, tb0 + 512)
    assert np.array_equal(kt[:, :tb0], layout.pack_k_tiles(u, d, n))
    assert np.array_equal(kt[0, tb0:].copy().view(np.float16).reshape(32, 8), m[0])      # [position][block]
    vt = layout.pack_v_tiles(u, d, n, m)
    assert np.array_equal(vt[:, :tb0], layout.pack_v_tiles(u, d, n))
    assert np.array_equal(vt[0, tb0:].copy().view(np.float16).reshape(8, 32), m[0].T)    # [block][position]
    lay0 = layout.slab_layout(_cfg(k_bits=n, v_bits=n))
    lay1 = layout.slab_layout(_cfg(k_bits=n, v_bits=n, v_min=1))
    assert lay1["v_body"][1] == lay0["v_body"][1] * (4 * n + 4) // (4 * n + 2)
    assert lay1["k_body"][1] == lay0["k_body"][1]
