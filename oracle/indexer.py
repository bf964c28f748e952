"""The QSA indexer: pooled index keys, scores and the selection of a budget of positions (oracle; test
infrastructure only).

The offload page ("You can offload most of Qwen3.8-Flash-Next's KV cache to RAM ...", QSA paragraph and the
paragraph on what must stay on the GPU) fixes the shape of the step that feeds sparse decode: a cheap indexer
runs over pooled, compressed keys, the pooled width being indexer_head_dim = 128 divided by
indexer_compress_ratio = 4; the indexer picks at most indexer_budget = 2,048 positions, and the layer then reads
only the main-KV rows at those positions. What stays resident per token and layer is the pooled index key,
1 x (128 / 4) x 2 bytes = 64 bytes, plus a 2-byte slot: 66 bytes against a full bf16 row of 2,048 bytes.

Readings (the page gives the sizes, not the arithmetic):

* Pooling: the 128-value indexer key of a token (bf16; it comes from the model's indexer projection, which the
  page does not give) is pooled by the mean of each group of `ratio` consecutive values: summed in fp32 in
  order, multiplied by 1/ratio (exact: ratio is a power of two), rounded to bf16 with round to nearest even.
  One index head per layer (the page's "1 x").
* The 2-byte slot locates a token's main-KV row when that row is host-resident; a cache whose rows sit in HBM at
  their position needs no slot, so the stored index entry is the 64-byte pooled key.
* Score of position t for an index query q (32 bf16 values, in the pooled width): the sum over i = 0..31 of
  q_i * k_ti, each product exact in fp32 (8 + 8 significant bits) and the sum accumulated in fp32 in channel
  order (the page fixes no precision; this is the GPU kernel's). A zero score is +0.
* Selection: the newest n_recent positions are always taken; of the older positions, the budget - n_recent with
  the highest scores, equal scores going to the lower position. With no more than the budget positions in the
  sequence, all are taken. The list is returned in ascending position order, padded with -1 (an entry sparse
  decode skips) when the sequence holds fewer positions than the budget.
"""
from __future__ import annotations

import numpy as np

POOLED = 32          # pooled width: indexer_head_dim / indexer_compress_ratio = 128 / 4
KEY_BYTES = 2 * POOLED


def index_token_bytes(head_dim: int = 128, ratio: int = 4, n_heads: int = 1) -> int:
    """Bytes of one token's pooled index key: n_heads x (head_dim / ratio) x 2 bytes."""
    return n_heads * (head_dim // ratio) * 2


def _bf16_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _f32_to_bf16_rne(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def pool_keys(key_bits: np.ndarray, ratio: int = 4) -> np.ndarray:
    """bf16 indexer keys [n, ratio * 32] -> pooled bf16 keys [n, 32]: the fp32 mean of each group of `ratio`
    consecutive values (summed in order), rounded to bf16."""
    assert ratio in (1, 2, 4, 8, 16)
    x = _bf16_f32(key_bits)
    n, width = x.shape
    assert width == ratio * POOLED
    g = x.reshape(n, POOLED, ratio)
    s = g[:, :, 0].copy()
    for j in range(1, ratio):
        s = (s + g[:, :, j]).astype(np.float32)          # fp32 addition, in order
    mean = (s * np.float32(1.0 / ratio)).astype(np.float32)   # exact: a power of two
    return _f32_to_bf16_rne(mean)


def scores(query_bits: np.ndarray, pooled_bits: np.ndarray) -> np.ndarray:
    """fp32 scores [n] of pooled keys [n, 32] against one query [32]: products exact in fp32, summed in channel
    order in fp32; -0 becomes +0."""
    q = _bf16_f32(query_bits)
    k = _bf16_f32(pooled_bits)
    acc = np.zeros(k.shape[0], dtype=np.float32)
    for i in range(POOLED):
        acc = (acc + (q[i] * k[:, i]).astype(np.float32)).astype(np.float32)
    return acc + np.float32(0.0)                          # -0 + 0 = +0


def select(score: np.ndarray, length: int, budget: int, n_recent: int = 0) -> np.ndarray:
    """Positions chosen from a sequence of `length` positions whose first length - n_recent have `score`:
    the newest n_recent, then the highest scores of the rest (equal scores: lower position first); ascending,
    padded with -1 to `budget` entries."""
    assert 0 <= n_recent <= budget
    m = max(length - n_recent, 0)
    recent = np.arange(m, length, dtype=np.int64)
    k = budget - len(recent)
    if m <= k:
        chosen = np.arange(m, dtype=np.int64)
    else:
        pos = np.arange(m, dtype=np.int64)
        order = np.lexsort((pos, -np.asarray(score[:m], dtype=np.float64)))   # score descending, then position
        chosen = np.sort(order[:k])
    out = np.full(budget, -1, dtype=np.int32)
    sel = np.concatenate([chosen, recent])
    out[:len(sel)] = sel
    return out
