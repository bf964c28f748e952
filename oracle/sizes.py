"""Algorithmic bytes read by one decode call (oracle; test infrastructure only).

The offload page counts the bytes a step reads: a bf16 QSA row is 2 KV heads x
256 x (K and V) x 2 bytes = 2,048 bytes per token per layer, so a budget of 2,048
positions reads 4 MiB per layer (offload page, byte arithmetic and QSA paragraph).
The same count applies to a quantized cache with the row size of its format
(BeeLlama.cpp v0.4.1 page, KV MiB column: N bits per value plus one fp16 scale per
32 values; a qN_1 type adds one fp16 minimum per 32 values, KVarN benchmark page,
cache-size column of q5_1 and q8_0-q5_1).

A call's algorithmic bytes are the rows it must read (every attended position's K
and V row of each KV head, from the body or the ring), the KVarN scales of each
sequence, the bf16 query rows it reads and the fp32 output rows it writes; the
split partials and any repeated read are not counted.
"""
from __future__ import annotations

from .layout import row_bytes  # noqa: F401  (re-exported)


def kv_token_bytes(n_bits_k: int, n_bits_v: int, n_kv_heads: int, head_dim: int, k_min: bool = False,
                   v_min: bool = False) -> int:
    """Bytes of one token in one layer: every KV head, K and V (a qN_1 side adds an fp16 minimum per block)."""
    return n_kv_heads * (row_bytes(n_bits_k, head_dim, k_min) + row_bytes(n_bits_v, head_dim, v_min))


def ring_token_bytes(tail_dtype: int, n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one ring token in one layer: bf16 or f16 values (tail dtypes 1 and 3), or q8_0 rows (2)."""
    if tail_dtype in (1, 3):   # bf16 or f16 values: 2 bytes each
        return n_kv_heads * 2 * head_dim * 2
    if tail_dtype == 2:
        return n_kv_heads * 2 * row_bytes(8, head_dim)
    return 0


def decode_kv_bytes(cfg: dict, lengths, body_lengths) -> int:
    """Cache bytes one dense decode call reads: body rows + ring rows (+ the KVarN scales per sequence)."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    body = kv_token_bytes(cfg["k_bits"], cfg["v_bits"], hk, d, bool(cfg.get("k_min", 0)), bool(cfg.get("v_min", 0)))
    ring = ring_token_bytes(cfg["tail_dtype"] if cfg["tail_len"] > 0 else 0, hk, d)
    total = 0
    for ln, bl in zip(lengths, body_lengths):
        total += bl * body + (ln - bl) * ring
        if cfg["kvarn"]:
            total += hk * 2 * d * 2
    return total


def query_out_bytes(cfg: dict, n_queries: int) -> int:
    """bf16 query rows read and fp32 output rows written by a call over n_queries query vectors."""
    return n_queries * cfg["n_q_heads"] * cfg["head_dim"] * (2 + 4)


def decode_bytes(cfg: dict, lengths, body_lengths) -> int:
    """Algorithmic bytes of one dense decode call (one query per sequence)."""
    return decode_kv_bytes(cfg, lengths, body_lengths) + query_out_bytes(cfg, len(lengths))


def sparse_kv_bytes(cfg: dict, n_body: int, n_ring: int) -> int:
    """Cache bytes of a sparse read of n_body body positions and n_ring ring positions."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    return (n_body * kv_token_bytes(cfg["k_bits"], cfg["v_bits"], hk, d, bool(cfg.get("k_min", 0)),
                                    bool(cfg.get("v_min", 0)))
            + n_ring * ring_token_bytes(cfg["tail_dtype"] if cfg.get("tail_len", 0) > 0 else 0, hk, d))


def sparse_bytes(cfg: dict, n_body: int, n_ring: int) -> int:
    """Cache bytes of a sparse read (kept as the name the pins use)."""
    return sparse_kv_bytes(cfg, n_body, n_ring)


def bf16_token_bytes(n_kv_heads: int, head_dim: int) -> int:
    """Unquantized bf16 K+V bytes of one token in one layer."""
    return n_kv_heads * head_dim * 2 * 2
