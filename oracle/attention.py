"""Exact softmax attention over dequantized cache values, in fp64 (oracle).

Test infrastructure only. Decode attention reads every cached position of a
full-attention layer each step (offload page: decode is a bandwidth problem;
full-attention layers read the whole KV cache every step). A QSA layer reads only
the main-KV rows at the positions its indexer chose, so the indexer budget, not
the context, bounds the bytes (offload page, QSA paragraph).

Readings: the softmax scale defaults to 1/sqrt(D); q arrives already rotated and
K is stored post-rotation; no mask beyond the sequence length; grouped-query
attention maps query head h to KV head floor(h / (Hq / Hkv)). The softmax is the
plain two-pass definition: m = max s, w = exp(s - m), out = sum w V / sum w.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """q [Hq, D] fp64, k/v [T, Hkv, D] fp64 -> out [Hq, D] fp64."""
    hq = q.shape[0]
    hk = k.shape[1]
    group = hq // hk
    out = np.zeros_like(q, dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = scale * (k[:, g, :] @ q[h])                 # [T]
        m = np.max(s)
        w = np.exp(s - m)
        out[h] = (w @ v[:, g, :]) / np.sum(w)
    return out


def _q64(q_bits: np.ndarray) -> np.ndarray:
    return (np.asarray(q_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _scale(cache, scale):
    return 1.0 / np.sqrt(cache.cfg["head_dim"]) if (scale is None or scale <= 0) else float(scale)


def decode_reference(cache, layer: int, seq_ids, q_bits: np.ndarray, scale=None) -> np.ndarray:
    """Dense decode over positions [0, len) of each sequence: out [n_seqs, Hq, D] fp64."""
    sc = _scale(cache, scale)
    out = []
    for i, sid in enumerate(seq_ids):
        k, v = cache.dequantized(layer, sid)
        out.append(attend(_q64(q_bits[i]), k, v, sc))
    return np.stack(out)


def sparse_reference(cache, layer: int, seq_ids, q_bits: np.ndarray, positions: np.ndarray,
                     scale=None) -> np.ndarray:
    """Attention over positions[i] (list order; one list per sequence, shared by all KV heads).

    Reading (the pages say only that the layer reads the rows the indexer chose): an entry
    outside [0, len) names no row and is skipped; a repeated entry is attended as often as it
    appears; a list with no valid entry gives a zero output."""
    sc = _scale(cache, scale)
    out = []
    for i, sid in enumerate(seq_ids):
        n, _ = cache.lengths(layer, sid)
        pos = np.asarray(positions[i], dtype=np.int64)
        pos = pos[(pos >= 0) & (pos < n)]
        if len(pos) == 0:
            out.append(np.zeros((q_bits.shape[1], cache.cfg["head_dim"])))
            continue
        k, v = cache.dequantized(layer, sid, pos)
        out.append(attend(_q64(q_bits[i]), k, v, sc))
    return np.stack(out)


def multi_query_reference(cache, layer: int, seq_ids, q_bits: np.ndarray, scale=None) -> np.ndarray:
    """Decode of T = 1 + k queries per sequence at once, as in verifying k drafted tokens (Qwen3.8-27B page,
    decode-speed paragraph: the engine drafts up to 7 tokens per step with MTP heads). q_bits [n_seqs, T, Hq, D]
    bf16 bits -> out [n_seqs, T, Hq, D] fp64.

    Reading (the pages do not spell out the verification step): the T tokens are the last T positions already in
    the cache; query t sits at position len - T + t and, causally, attends to positions 0 .. len - T + t."""
    sc = _scale(cache, scale)
    n_q = q_bits.shape[1]
    out = np.zeros(q_bits.shape, dtype=np.float64)
    for i, sid in enumerate(seq_ids):
        n, _ = cache.lengths(layer, sid)
        if n < n_q:
            raise ValueError(f"sequence {sid} holds {n} positions, fewer than {n_q} queries")
        k, v = cache.dequantized(layer, sid)              # positions 0 .. n-1
        for t in range(n_q):
            end = n - n_q + t + 1                         # query t attends to positions [0, end)
            out[i, t] = attend(_q64(q_bits[i, t]), k[:end], v[:end], sc)
    return out


def prefill_reference(cache, layer: int, seq_ids, n_new, q_bits: np.ndarray, rows=None, scale=None) -> np.ndarray:
    """Attention of the queries of a prefill chunk that has just been appended (the KVarN benchmark page and the
    Qwen3.8-27B page measure prompt processing per cache type). q_bits [sum n_new, Hq, D] bf16 bits, sequences
    packed in call order -> out [len(rows), Hq, D] fp64 for the packed rows ``rows`` (all rows by default).

    Reading (the pages give prefill timings only): the query of new token j of sequence i sits at position
    len_i - n_i + j (len_i: the length after the append) and attends causally to positions 0 .. len_i - n_i + j
    through the cache as it stands after the append, i.e. through the stored representation of every position,
    the chunk's own included."""
    sc = _scale(cache, scale)
    n_new = [int(x) for x in n_new]
    total = sum(n_new)
    rows = np.arange(total) if rows is None else np.asarray(rows, dtype=np.int64)
    owner = np.repeat(np.arange(len(seq_ids)), n_new)            # packed row -> index into seq_ids
    first = np.concatenate([[0], np.cumsum(n_new)])[:-1]
    out = np.zeros((len(rows),) + q_bits.shape[1:], dtype=np.float64)
    kv = {}
    for r_i, row in enumerate(rows):
        i = int(owner[row])
        sid = seq_ids[i]
        if sid not in kv:
            kv[sid] = cache.dequantized(layer, sid)
        k, v = kv[sid]
        n, _ = cache.lengths(layer, sid)
        end = n - n_new[i] + (row - first[i]) + 1                 # attends to positions [0, end)
        out[r_i] = attend(_q64(q_bits[row]), k[:end], v[:end], sc)
    return out
