"""Pins of the oracle's cache state machine: tail, ring, eviction and KVarN.

The special cases come from the pages: a precision tail stores the newest tokens
without loss (BeeLlama.cpp v0.4.1 page); with a context shorter than the 8-bit
ring window the output equals a q8_0 cache (Qwen3.8-27B page). The rest are
invariants of the semantics: chunk invariance, the ring holding exactly the newest
W after an evict, W = 0 meaning no ring.
"""
import numpy as np
import pytest

from oracle import OracleCache, quant
from oracle.layout import slab_layout
from workloads import small_tokens, bf16_to_f32


def cfg(**kw):
    c = dict(n_layers=1, max_seqs=2, capacity=512, n_q_heads=4, n_kv_heads=2, head_dim=256,
             k_bits=6, v_bits=5, kvarn=0, tail_len=64, tail_slack=32, tail_dtype=1)
    c.update(kw)
    return c


def _append_all(c, k, v, chunks, seq=0, evict_after=()):
    o = OracleCache(c)
    off = 0
    for idx, n in enumerate(chunks):
        o.append(0, [seq], [n], k[off:off + n], v[off:off + n])
        off += n
        if idx in evict_after:
            o.tail_evict(0, [seq])
    return o


def test_tail_is_lossless_below_window():
    c = cfg(tail_len=128, tail_slack=32)
    k, v = small_tokens(1, 100, 2, 256)
    o = _append_all(c, k, v, [37, 63])
    kk, vv = o.dequantized(0, 0)
    assert o.lengths(0, 0) == (100, 0)
    assert np.array_equal(kk, bf16_to_f32(k).astype(np.float64))
    assert np.array_equal(vv, bf16_to_f32(v).astype(np.float64))


def test_q8_ring_below_window_equals_q8_body():
    k, v = small_tokens(2, 90, 2, 256, scale=np.full((2, 2, 256), 3.0, dtype=np.float32))
    ring = _append_all(cfg(tail_len=128, tail_slack=32, tail_dtype=2), k, v, [90])
    body = _append_all(cfg(tail_len=0, k_bits=8, v_bits=8), k, v, [90])
    a, b = ring.dequantized(0, 0), body.dequantized(0, 0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
@pytest.mark.parametrize("kvarn", [0, 1])
def test_chunk_invariance(tail_dtype, kvarn):
    c = cfg(tail_dtype=tail_dtype, kvarn=kvarn, tail_len=64, tail_slack=32)
    k, v = small_tokens(3, 300, 2, 256)
    first = 40          # KVarN calibrates on the first chunk: keep it fixed
    ref = _append_all(c, k, v, [first] + [1] * 260)
    for chunks, ev in (([first, 260], ()), ([first, 7, 100, 53, 100], (1, 3)), ([first] + [20] * 13, (5, 6, 9))):
        o = _append_all(c, k, v, chunks, evict_after=ev)
        o.tail_evict(0, [0])
        ref.tail_evict(0, [0])
        assert o.lengths(0, 0) == ref.lengths(0, 0) == (300, 300 - 64)
        a, b = o.dequantized(0, 0), ref.dequantized(0, 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        sa, sb = o.st(0, 0), ref.st(0, 0)
        bl = 300 - 64
        assert np.array_equal(sa.ku[:bl], sb.ku[:bl]) and np.array_equal(sa.vd[:bl], sb.vd[:bl])


def test_append_evicts_only_on_overflow_and_evict_drains_to_window():
    c = cfg(tail_len=64, tail_slack=32)     # R = 96
    k, v = small_tokens(4, 400, 2, 256)
    o = OracleCache(c)
    o.append(0, [0], [50], k[:50], v[:50])
    assert o.lengths(0, 0) == (50, 0)
    o.append(0, [0], [40], k[50:90], v[50:90])
    assert o.lengths(0, 0) == (90, 0)       # 90 <= R: nothing leaves
    o.append(0, [0], [20], k[90:110], v[90:110])
    assert o.lengths(0, 0) == (110, 14)     # overflow: the oldest 14 leave
    o.tail_evict(0, [0])
    assert o.lengths(0, 0) == (110, 46)     # drained to the newest 64
    o.tail_evict(0, [0])
    assert o.lengths(0, 0) == (110, 46)
    o.append(0, [0], [290], k[110:400], v[110:400])
    assert o.lengths(0, 0) == (400, 400 - 96)


@pytest.mark.parametrize("tail_dtype", [1, 2, 3])
def test_evicted_rows_are_requantized_ring_values(tail_dtype):
    c = cfg(tail_len=64, tail_slack=32, tail_dtype=tail_dtype)
    k, v = small_tokens(5, 200, 2, 256)
    o = _append_all(c, k, v, [100, 100])
    o.tail_evict(0, [0])
    s = o.st(0, 0)
    kx = bf16_to_f32(k[:136])
    if tail_dtype == 2:
        u8, d8 = quant.quantize_blocks(kx, 8)
        kx = quant.dequantize_blocks(u8, d8, 8).astype(np.float32)
    if tail_dtype == 3:   # the f16 value (numpy's IEEE binary16 conversion, round to nearest even)
        kx = kx.astype(np.float16).astype(np.float32)
    u, d = quant.quantize_blocks(kx, 6)
    assert np.array_equal(s.ku[:136], u) and np.array_equal(s.kd[:136].view(np.uint16), d.view(np.uint16))


def test_zero_window_is_no_ring():
    k, v = small_tokens(6, 120, 2, 256)
    a = _append_all(cfg(tail_len=0, tail_slack=0), k, v, [60, 60])
    b = _append_all(cfg(tail_len=0, tail_slack=512, tail_dtype=2), k, v, [120])
    assert a.lengths(0, 0) == b.lengths(0, 0) == (120, 120)
    assert np.array_equal(a.dequantized(0, 0)[0], b.dequantized(0, 0)[0])
    lay = slab_layout(cfg(tail_len=0, tail_slack=512, tail_dtype=2))
    assert lay["k_ring"][1] == 0 and lay["v_ring"][1] == 0


def test_kvarn_unit_rms_equals_plain():
    # first chunk with every channel of RMS exactly 1 (values +-1) -> sigma = 1
    n = 32
    signs = np.where(np.random.default_rng(0).random((n, 2, 256)) < 0.5, -1.0, 1.0).astype(np.float32)
    from workloads import bf16_bits
    kb = bf16_bits(signs)
    k2, v2 = small_tokens(7, 100, 2, 256)
    k = np.concatenate([kb, k2])
    v = np.concatenate([kb, v2])
    a = _append_all(cfg(kvarn=1, tail_len=0), k, v, [n, 100])
    b = _append_all(cfg(kvarn=0, tail_len=0), k, v, [n, 100])
    assert np.all(a.st(0, 0).sigma.astype(np.float32) == 1.0)
    assert np.array_equal(a.st(0, 0).ku, b.st(0, 0).ku)
    assert np.array_equal(a.st(0, 0).vd.view(np.uint16), b.st(0, 0).vd.view(np.uint16))


def test_kvarn_dequant_includes_sigma():
    sc = np.ones((2, 2, 256), dtype=np.float32)
    sc[:, :, 3] = 16.0
    k, v = small_tokens(8, 64, 2, 256, scale=sc)
    o = _append_all(cfg(kvarn=1, tail_len=0), k, v, [64])
    s = o.st(0, 0)
    kk, _ = o.dequantized(0, 0)
    y = quant.normalize(bf16_to_f32(k), s.sigma[:, 0, :])
    u, d = quant.quantize_blocks(y, 6)
    expect = quant.dequantize_blocks(u, d, 6) * s.sigma[:, 0, :].astype(np.float64)
    assert np.array_equal(kk, expect)
    # the per-channel scale tracks the channel's RMS: the x16 channel gets sigma ~ 16
    assert np.all(np.abs(s.sigma[:, 0, 3].astype(np.float64) / 16.0 - 1) < 0.35)


def test_capacity_is_enforced():
    o = OracleCache(cfg(capacity=64, tail_len=0))
    k, v = small_tokens(9, 65, 2, 256)
    o.append(0, [0], [64], k[:64], v[:64])
    with pytest.raises(ValueError):
        o.append(0, [0], [1], k[64:], v[64:])


def test_sequences_are_independent():
    c = cfg()
    k, v = small_tokens(10, 150, 2, 256)
    o = OracleCache(c)
    o.append(0, [1, 0], [100, 50], k, v)
    a = _append_all(c, k[:100], v[:100], [100], seq=1)
    b = _append_all(c, k[100:], v[100:], [50], seq=0)
    assert np.array_equal(o.dequantized(0, 1)[0], a.dequantized(0, 1)[0])
    assert np.array_equal(o.dequantized(0, 0)[1], b.dequantized(0, 0)[1])


# bf16 input bits -> IEEE binary16 bits, worked out from the two formats' definitions (1 sign, 8 / 5 exponent
# bits with bias 127 / 15, 7 / 10 mantissa bits; f16 subnormals are multiples of 2^-24; ties to even)
F16_CASES = [
    (0x3F80, 0x3C00),   # 1.0
    (0xC020, 0xC100),   # -2.5 = -1.25 * 2^1: exponent 16, mantissa 256
    (0x477F, 0x7BF8),   # 65280 = 1.9921875 * 2^15: exponent 30, mantissa 1016
    (0x4780, 0x7C00),   # 65536: above the largest f16 (65504) -> +infinity
    (0x3580, 0x0010),   # 2^-20 = 16 * 2^-24: subnormal
    (0x3300, 0x0000),   # 2^-25: half of 2^-24, tie -> even (zero)
    (0x33C0, 0x0002),   # 1.5 * 2^-24: tie between 1 and 2 ulps -> even (2)
    (0x3340, 0x0001),   # 0.75 * 2^-24 -> 1 ulp
]


def test_f16_tail_stores_ieee_binary16_of_the_input():
    """F16 precision tail (BeeLlama.cpp v0.4.1 page: recent tokens kept in BF16 or F16): the ring holds the
    binary16 rounding of each bf16 input value."""
    c = cfg(tail_len=64, tail_slack=32, tail_dtype=3)
    k = np.zeros((len(F16_CASES), 2, 256), dtype=np.uint16)
    v = np.zeros_like(k)
    for i, (b, _) in enumerate(F16_CASES):
        k[i, :, 3 * i] = b
        v[i, 1, 7] = b
    o = _append_all(c, k, v, [len(F16_CASES)])
    s = o.st(0, 0)
    for i, (_, want) in enumerate(F16_CASES):
        assert s.rk[i, 0, 3 * i] == want and s.rk[i, 1, 3 * i] == want, (hex(F16_CASES[i][0]), hex(s.rk[i, 0, 3 * i]))
        assert s.rv[i, 1, 7] == want


def test_f16_tail_below_window_holds_the_rounded_inputs():
    """Below the window nothing is quantized: the f16 cache holds exactly the binary16 values of the inputs
    (numpy's IEEE conversion), including inputs in the f16 subnormal range, where the rounding shows."""
    c = cfg(tail_len=128, tail_slack=32, tail_dtype=3)
    k, v = small_tokens(8, 100, 2, 256, scale=np.full((2, 2, 256), 4.0, dtype=np.float32))
    k[:, 0, 0] = 0x3581   # 2^-20 * (1 + 2^-7) = 16.125 * 2^-24 -> 16 * 2^-24 in f16
    o = _append_all(c, k, v, [60, 40])
    kk, vv = o.dequantized(0, 0)
    k16 = bf16_to_f32(k).astype(np.float16).astype(np.float64)
    v16 = bf16_to_f32(v).astype(np.float16).astype(np.float64)
    assert np.array_equal(kk, k16) and np.array_equal(vv, v16)
    assert np.all(kk[:, 0, 0] == 16 * 2.0 ** -24)


@pytest.mark.parametrize("tail_dtype,kvarn", [(1, 0), (2, 1), (3, 0)])
def test_truncate_then_append_equals_never_appending_the_dropped(tail_dtype, kvarn):
    """Rolling back rejected drafts: append drafts, truncate, append the accepted tokens, step on; every length,
    dequantized value and attention output equals a cache that only ever saw the accepted tokens."""
    import oracle
    from workloads import small_query
    c = dict(n_layers=1, max_seqs=1, capacity=512, n_q_heads=4, n_kv_heads=2, head_dim=256, k_bits=5,
             v_bits=3, kvarn=kvarn, tail_len=16, tail_slack=16, tail_dtype=tail_dtype)
    k, v = small_tokens(40 + tail_dtype, 300, 2, 256)
    a, b = OracleCache(c), OracleCache(c)
    a.append(0, [0], [100], k[:100], v[:100])
    b.append(0, [0], [100], k[:100], v[:100])
    a.tail_evict(0, [0])
    b.tail_evict(0, [0])
    off = 100
    for drafts, accepted in ((7, 3), (4, 0), (7, 7), (2, 1)):
        a.append(0, [0], [drafts], k[200:200 + drafts], v[200:200 + drafts])   # drafts that will be rejected
        n, _ = a.lengths(0, 0)
        a.truncate(0, [0], [n - drafts])
        a.append(0, [0], [accepted], k[off:off + accepted], v[off:off + accepted])
        b.append(0, [0], [accepted], k[off:off + accepted], v[off:off + accepted])
        off += accepted
        a.tail_evict(0, [0])
        b.tail_evict(0, [0])
        assert a.lengths(0, 0) == b.lengths(0, 0)
        ka, va = a.dequantized(0, 0)
        kb, vb = b.dequantized(0, 0)
        np.testing.assert_array_equal(ka, kb)
        np.testing.assert_array_equal(va, vb)
        q = small_query(off, 1, 4, 256)
        np.testing.assert_array_equal(oracle.decode_reference(a, 0, [0], q), oracle.decode_reference(b, 0, [0], q))


def test_truncate_keeps_to_the_ring():
    c = dict(n_layers=1, max_seqs=1, capacity=256, n_q_heads=4, n_kv_heads=2, head_dim=256, k_bits=4,
             v_bits=4, kvarn=0, tail_len=16, tail_slack=16, tail_dtype=1)
    k, v = small_tokens(3, 60, 2, 256)
    o = OracleCache(c)
    o.append(0, [0], [60], k, v)
    o.tail_evict(0, [0])
    n, body = o.lengths(0, 0)
    with pytest.raises(ValueError):
        o.truncate(0, [0], [body - 1])
    with pytest.raises(ValueError):
        o.truncate(0, [0], [n + 1])
    o.truncate(0, [0], [body])
    assert o.lengths(0, 0) == (body, body)


@pytest.mark.parametrize("k_min,v_min,tail_dtype", [(1, 0, 0), (0, 1, 1), (1, 1, 2), (1, 1, 3)])
def test_qn1_body_reproduces_values_on_its_grid(k_min, v_min, tail_dtype):
    """Inputs that lie on a power-of-two grid with an offset (every block spanning all 2^N levels) are stored
    exactly by a qN_1 side, through the ring and after eviction; a qN_0 side keeps its own rounding."""
    nk, nv = 4, 3
    n = 100
    rng = np.random.default_rng(7 + 4 * k_min + 2 * v_min + tail_dtype)

    def grid(bits, off, k):
        c = rng.integers(0, 1 << bits, size=(n, 2, 8, 32))
        c[..., 0] = 0
        c[..., 1] = (1 << bits) - 1
        return ((c + off) * 2.0 ** k).reshape(n, 2, 256).astype(np.float32)

    kx, vx = grid(nk, -5, -3), grid(nv, 2, 1)
    from workloads import bf16_bits
    kb, vb = bf16_bits(kx), bf16_bits(vx)
    assert np.array_equal(bf16_to_f32(kb), kx) and np.array_equal(bf16_to_f32(vb), vx)   # exact in bf16
    cfg = dict(n_layers=1, max_seqs=1, capacity=256, n_q_heads=4, n_kv_heads=2, head_dim=256, k_bits=nk,
               v_bits=nv, kvarn=0, tail_len=16 if tail_dtype else 0, tail_slack=16, tail_dtype=tail_dtype,
               k_min=k_min, v_min=v_min)
    o = OracleCache(cfg)
    o.append(0, [0], [60], kb[:60], vb[:60])
    o.tail_evict(0, [0])
    o.append(0, [0], [40], kb[60:], vb[60:])
    o.tail_evict(0, [0])
    n_len, body = o.lengths(0, 0)
    assert n_len == n and (body == n if not tail_dtype else body == n - 16)
    k, v = o.dequantized(0, 0)
    below = np.arange(body)
    if tail_dtype == 2:   # body rows went through the q8_0 ring first: only their own grid survives exactly
        return
    if k_min:
        assert np.array_equal(k[below], kx[below].astype(np.float64))
    else:
        assert not np.array_equal(k[below], kx[below].astype(np.float64))
    if v_min:
        assert np.array_equal(v[below], vx[below].astype(np.float64))
    lay = slab_layout(cfg)
    img = o.slab_image(0, 0)
    assert img.shape[0] == lay["slab"]


# ---- token-axis K (a block is the 32 positions of one channel in a position tile)

def _tok_cfg(**kw):
    c = dict(n_layers=1, max_seqs=1, capacity=512, n_q_heads=4, n_kv_heads=2, head_dim=256, k_bits=4, v_bits=5,
             kvarn=0, tail_len=40, tail_slack=56, tail_dtype=1, k_axis=1)
    c.update(kw)
    return c


def test_token_axis_k_stores_per_channel_grids_exactly():
    """K values that are, per (tile, channel), integer codes times a channel-specific power of two spanning the
    full code range are stored exactly along the token axis, though every position mixes 256 different scales
    (which a per-token block of 32 channels could not represent exactly)."""
    rng = np.random.default_rng(5)
    n = 192
    qmax = 7
    c = rng.integers(-qmax, qmax + 1, size=(n // 32, 32, 2, 256))
    c[:, 3] = qmax
    c[:, 9] = -qmax
    ex = rng.integers(-6, 4, size=(n // 32, 1, 2, 256))
    kx = (c * 2.0 ** ex).reshape(n, 2, 256).astype(np.float32)
    from workloads import bf16_bits
    kb = bf16_bits(kx)
    assert np.array_equal(bf16_to_f32(kb), kx)
    _, vb = small_tokens(9, n, 2, 256)
    o = OracleCache(_tok_cfg(tail_dtype=1))
    o.append(0, [0], [n], kb, vb)
    o.tail_evict(0, [0])
    ln, body = o.lengths(0, 0)
    assert body == (n - 40) // 32 * 32 == 128
    k, _ = o.dequantized(0, 0, np.arange(body))
    assert np.array_equal(k, kx[:body].astype(np.float64))
    per_token = OracleCache(_tok_cfg(k_axis=0, tail_len=0, tail_slack=0, tail_dtype=0))
    per_token.append(0, [0], [n], kb, vb)
    k2, _ = per_token.dequantized(0, 0, np.arange(body))
    assert not np.array_equal(k2, kx[:body].astype(np.float64))


@pytest.mark.parametrize("k_min,tail_dtype", [(0, 1), (1, 2), (0, 3), (1, 1)])
def test_token_axis_body_grows_by_whole_tiles_and_is_chunk_invariant(k_min, tail_dtype):
    k, v = small_tokens(21 + tail_dtype, 300, 2, 256)
    cfg = _tok_cfg(k_min=k_min, tail_dtype=tail_dtype)
    a = OracleCache(cfg)
    a.append(0, [0], [300], k, v)
    a.tail_evict(0, [0])
    b = OracleCache(cfg)
    off = 0
    for n in (1, 37, 90, 3, 64, 105):
        b.append(0, [0], [n], k[off:off + n], v[off:off + n])
        off += n
        ln, body = b.lengths(0, 0)
        assert body % 32 == 0 and ln - body <= cfg["tail_len"] + cfg["tail_slack"]
        if n <= 3:
            b.tail_evict(0, [0])
            ln, body = b.lengths(0, 0)
            assert cfg["tail_len"] <= ln - body < cfg["tail_len"] + 32 or ln < cfg["tail_len"]
    b.tail_evict(0, [0])
    assert a.lengths(0, 0) == b.lengths(0, 0)
    ka, va = a.dequantized(0, 0)
    kb2, vb2 = b.dequantized(0, 0)
    assert np.array_equal(ka, kb2) and np.array_equal(va, vb2)
    bl = a.lengths(0, 0)[1]
    sa, sb = a.st(0, 0), b.st(0, 0)
    assert np.array_equal(sa.ku[:bl], sb.ku[:bl]) and np.array_equal(sa.ktd[:bl // 32], sb.ktd[:bl // 32])
    # the body's K is within half a channel scale of the ring representation of the input
    ln, body = a.lengths(0, 0)
    kin = bf16_to_f32(k[:body]).astype(np.float64)
    if tail_dtype == 2:
        return
    st = a.st(0, 0)
    d = np.repeat(st.ktd[:body // 32].astype(np.float64), 32, axis=0)      # [pos, head, ch]
    extra = 0 if not k_min else np.abs(np.repeat(st.ktm[:body // 32].astype(np.float64), 32, axis=0)
                                       - kin.reshape(-1, 32, 2, 256).min(axis=1).repeat(32, axis=0))
    assert np.all(np.abs(ka[:body] - kin) <= d / 2 + extra + 2.0 ** -22 * (np.abs(kin) + 1))
