"""Seeded synthetic inputs for the quantized KV cache and its decode attention.

This module only draws random numbers and rounds them to bfloat16 storage; it
holds none of the cache's arithmetic (no quantizer, no layout, no attention).
Both the CPU oracle and the GPU path consume exactly the arrays produced here.

The five workloads stand in for the pages' real models and text (a Qwen-next
style model with 16 full-attention layers of 2 KV heads x 256, and a sparse
QSA layer stack of 12 layers with a 2048-position indexer budget), which are not
available: shapes follow the pages, values are Gaussian with the channel-scale
structure each workload names.

Every draw uses ``numpy.random.default_rng(SeedSequence([0, cfg, layer, seq,
chunk, kind]))`` so any slice of any workload can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

CHUNK = 4096            # prefill chunk length (tokens)
DECODE_BASE = 1 << 20   # chunk ids >= this are decode-step tokens
KIND_K, KIND_V, KIND_Q, KIND_SCALE, KIND_POS, KIND_LEN, KIND_OUTLIER, KIND_IKEY, KIND_IQ = range(9)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Expand bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, *[int(k) for k in key]]))


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: cache shape, cache format and the value recipe."""
    cfg: int
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    k_bits: int
    v_bits: int
    kvarn: int
    tail_len: int
    tail_slack: int
    tail_dtype: int           # 0 none, 1 bf16, 2 q8_0
    contexts: Sequence[int]   # prefill length per sequence
    decode_steps: int
    budget: int = 0           # sparse positions per step (0 = dense decode)
    recent: int = 0           # of the budget, this many newest positions
    capacity: int = 0         # positions per sequence the cache is sized for
    layout: int = 0           # 0: V tiles (dense decode), 1: rows (sparse decode)

    def cache_config(self, capacity: Optional[int] = None) -> dict:
        cap = capacity if capacity is not None else self.capacity
        return dict(n_layers=self.n_layers, max_seqs=self.batch, capacity=cap,
                    n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, k_bits=self.k_bits, v_bits=self.v_bits,
                    kvarn=self.kvarn, tail_len=self.tail_len, tail_slack=self.tail_slack,
                    tail_dtype=self.tail_dtype, layout=self.layout)


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def _contexts_cfg3() -> List[int]:
    r = _rng(3, 0, 0, 0, KIND_LEN)
    return [int(v) for v in r.integers(16384, 65536 + 1, size=8)]


def workload(cfg: int, capacity_extra: int = 64) -> Workload:
    """The five synthetic workloads (cfg 1..5)."""
    if cfg == 1:
        return Workload(1, "q8_0 single layer, ctx 4096", 1, 1, 16, 2, 256, 8, 8, 0, 0, 0, 0,
                        [4096], 0, capacity=4096 + capacity_extra)
    if cfg == 2:
        return Workload(2, "K6/V5 + bf16 tail 2048, ctx 65536, 16 layers", 16, 1, 16, 2, 256, 6, 5, 0,
                        2048, 512, 1, [65536], 64, capacity=65536 + capacity_extra)
    if cfg == 3:
        ctx = _contexts_cfg3()
        return Workload(3, "KVarN K4/V4 + bf16 tail 1024, 8 streams ctx U[16k,64k], 16 layers", 16, 8, 16, 2,
                        256, 4, 4, 1, 1024, 512, 1, ctx, 32,
                        capacity=_round_up(max(ctx) + 32 + capacity_extra, 32))
    if cfg == 4:
        return Workload(4, "K6/V5 + q8_0 ring 2048, ctx 262144, 16 layers", 16, 1, 16, 2, 256, 6, 5, 0,
                        2048, 512, 2, [262143], 1, capacity=262144 + capacity_extra)
    if cfg == 5:
        return Workload(5, "sparse q8_0, budget 2048 of ctx 262144, 12 layers", 12, 1, 16, 2, 256, 8, 8, 0,
                        0, 0, 0, [262144], 64, budget=2048, recent=512,
                        capacity=262144 + capacity_extra, layout=1)
    raise ValueError(cfg)


def outlier_channels(cfg: int) -> np.ndarray:
    """The 4 K channels scaled x20 in cfgs 1 and 4 (fixed for all tokens, heads and layers)."""
    r = _rng(cfg, 0, 0, 0, KIND_OUTLIER)
    return np.sort(r.choice(256, size=4, replace=False))


def channel_scales(cfg: int, layer: int, seq: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Per (head, K/V, channel) standard deviations, shape [Hkv, 2, D] float32."""
    r = _rng(cfg, layer, seq, 0, KIND_SCALE)
    if cfg == 2:
        # log-uniform in [0.1, 10]; the same for every sequence of a layer
        r = _rng(cfg, layer, 0, 0, KIND_SCALE)
        return (10.0 ** r.uniform(-1.0, 1.0, size=(n_kv_heads, 2, head_dim))).astype(np.float32)
    if cfg == 3:
        # heavy-tailed Student-t (nu = 3) channel scales
        return np.abs(r.standard_t(3, size=(n_kv_heads, 2, head_dim))).astype(np.float32)
    s = np.ones((n_kv_heads, 2, head_dim), dtype=np.float32)
    if cfg in (1, 4):
        s[:, 0, outlier_channels(cfg)] = 20.0
    return s


def kv_tokens(cfg: int, layer: int, seq: int, start: int, n: int, n_kv_heads: int = 2,
              head_dim: int = 256, chunk_id: Optional[int] = None):
    """K and V bf16 bit patterns [n, Hkv, D] for tokens [start, start + n) of one (layer, seq).

    Tokens are drawn per prefill chunk (``start`` must be chunk-aligned unless ``chunk_id``
    names an explicit decode-step draw)."""
    sc = channel_scales(cfg, layer, seq, n_kv_heads, head_dim)
    if chunk_id is None:
        assert start % CHUNK == 0 and n <= CHUNK, (start, n)
        chunk_id = start // CHUNK
    rk = _rng(cfg, layer, seq, chunk_id, KIND_K)
    rv = _rng(cfg, layer, seq, chunk_id, KIND_V)
    k = rk.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32) * sc[None, :, 0, :]
    v = rv.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32) * sc[None, :, 1, :]
    return bf16_bits(k), bf16_bits(v)


def prefill_tokens(cfg: int, layer: int, seq: int, length: int, n_kv_heads: int = 2, head_dim: int = 256):
    """All prefill tokens of one (layer, seq), concatenated from 4096-token chunks."""
    ks, vs = [], []
    for s in range(0, length, CHUNK):
        k, v = kv_tokens(cfg, layer, seq, s, min(CHUNK, length - s), n_kv_heads, head_dim)
        ks.append(k)
        vs.append(v)
    return np.concatenate(ks), np.concatenate(vs)


def decode_token(cfg: int, layer: int, seq: int, step: int, n_kv_heads: int = 2, head_dim: int = 256):
    """The K/V token appended at decode step ``step``: [1, Hkv, D] bf16 bits each."""
    return kv_tokens(cfg, layer, seq, 0, 1, n_kv_heads, head_dim, chunk_id=DECODE_BASE + step)


def query(cfg: int, layer: int, seq: int, step: int, n_q_heads: int = 16, head_dim: int = 256) -> np.ndarray:
    """Decode query [Hq, D] bf16 bits, N(0, 1)."""
    r = _rng(cfg, layer, seq, DECODE_BASE + step, KIND_Q)
    return bf16_bits(r.standard_normal((n_q_heads, head_dim), dtype=np.float32))


def prefill_queries(cfg: int, layer: int, seq: int, start: int, n: int, n_q_heads: int = 16,
                    head_dim: int = 256) -> np.ndarray:
    """Queries of prefill tokens [start, start + n) of one (layer, seq): bf16 bits [n, Hq, D], N(0, 1), drawn
    per 4096-token chunk like kv_tokens (``start`` chunk-aligned)."""
    assert start % CHUNK == 0 and n <= CHUNK, (start, n)
    r = _rng(cfg, layer, seq, start // CHUNK, KIND_Q)
    return bf16_bits(r.standard_normal((n, n_q_heads, head_dim), dtype=np.float32))


def sparse_positions(cfg: int, layer: int, seq: int, step: int, length: int, budget: int,
                     recent: int) -> np.ndarray:
    """Budget of distinct positions in [0, length): the newest ``recent`` plus uniform draws
    without replacement from the rest (int32, in draw order)."""
    r = _rng(cfg, layer, seq, DECODE_BASE + step, KIND_POS)
    newest = np.arange(length - recent, length, dtype=np.int64)
    rest = r.choice(length - recent, size=budget - recent, replace=False)
    return np.concatenate([newest, rest]).astype(np.int32)


def small_tokens(seed: int, n: int, n_kv_heads: int, head_dim: int, scale=None, kind: int = 0):
    """Generic Gaussian K/V bf16 bits for tests: [n, Hkv, D] each (optionally scaled per channel)."""
    r = _rng(1000 + seed, kind, 0, 0, KIND_K)
    k = r.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32)
    v = r.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32)
    if scale is not None:
        sc = np.asarray(scale, dtype=np.float32)
        k = k * sc[..., 0, :]
        v = v * sc[..., 1, :]
    return bf16_bits(k), bf16_bits(v)


def small_query(seed: int, n_seqs: int, n_q_heads: int, head_dim: int, std: float = 1.0) -> np.ndarray:
    r = _rng(2000 + seed, 0, 0, 0, KIND_Q)
    return bf16_bits(std * r.standard_normal((n_seqs, n_q_heads, head_dim), dtype=np.float32))


def index_keys(cfg: int, layer: int, seq: int, start: int, n: int, dim: int = 128,
               chunk_id: Optional[int] = None) -> np.ndarray:
    """Indexer keys (the model's indexer projection, not on the pages: N(0, 1) stand-ins) of tokens
    [start, start + n) of one (layer, seq): bf16 bits [n, dim], drawn per prefill chunk like kv_tokens."""
    if chunk_id is None:
        assert start % CHUNK == 0 and n <= CHUNK, (start, n)
        chunk_id = start // CHUNK
    r = _rng(cfg, layer, seq, chunk_id, KIND_IKEY)
    return bf16_bits(r.standard_normal((n, dim), dtype=np.float32))


def index_query(cfg: int, layer: int, seq: int, step: int, width: int = 32) -> np.ndarray:
    """Index query of a decode step in the pooled width: bf16 bits [width], N(0, 1)."""
    r = _rng(cfg, layer, seq, DECODE_BASE + step, KIND_IQ)
    return bf16_bits(r.standard_normal(width, dtype=np.float32))
