"""Algorithmic bytes read by one decode call (oracle; test infrastructure only).

The offload page counts the bytes a step reads: a bf16 QSA row is 2 KV heads x
256 x (K and V) x 2 bytes = 2,048 bytes per token per layer, so a budget of 2,048
positions reads 4 MiB per layer (offload page, byte arithmetic and QSA paragraph).
The same count applies to a quantized cache with the row size of its format.
"""
from __future__ import annotations

from .layout import row_bytes  # noqa: F401  (re-exported)


def kv_token_bytes(n_bits_k: int, n_bits_v: int, n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one token in one layer: every KV head, K and V."""
    return n_kv_heads * (row_bytes(n_bits_k, head_dim) + row_bytes(n_bits_v, head_dim))


def ring_token_bytes(tail_dtype: int, n_kv_heads: int, head_dim: int) -> int:
    if tail_dtype in (1, 3):   # bf16 or f16 values: 2 bytes each
        return n_kv_heads * 2 * head_dim * 2
    if tail_dtype == 2:
        return n_kv_heads * 2 * row_bytes(8, head_dim)
    return 0


def decode_bytes(cfg: dict, lengths, body_lengths) -> int:
    """KV bytes one dense decode call reads: body rows + ring rows (+ KVarN sigma)."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    body = kv_token_bytes(cfg["k_bits"], cfg["v_bits"], hk, d)
    ring = ring_token_bytes(cfg["tail_dtype"], hk, d)
    total = 0
    for ln, bl in zip(lengths, body_lengths):
        total += bl * body + (ln - bl) * ring
        if cfg["kvarn"]:
            total += hk * 2 * d * 2
    return total


def sparse_bytes(cfg: dict, n_body: int, n_ring: int) -> int:
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    return (n_body * kv_token_bytes(cfg["k_bits"], cfg["v_bits"], hk, d)
            + n_ring * ring_token_bytes(cfg["tail_dtype"], hk, d))


def bf16_token_bytes(n_kv_heads: int, head_dim: int) -> int:
    """Unquantized bf16 K+V bytes of one token in one layer."""
    return n_kv_heads * head_dim * 2 * 2
