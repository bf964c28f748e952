"""Thin Python binding of the kvq C ABI (include/kvq.h).

Argument marshalling only: every step of the cache and of attention runs in the HIP library
(``libkvq.so`` next to this file). PyTorch provides device memory (tensors' ``data_ptr()``) and streams
(``torch.cuda.current_stream().cuda_stream``). If the library is missing this module raises at import.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_E_INVALID, KVQ_E_CAPACITY, KVQ_E_SIZE, KVQ_E_HIP, KVQ_E_STATE = 0, -1, -2, -3, -4, -5
KVQ_MAX_BATCH, KVQ_MAX_QUERIES = 64, 8
TAIL_NONE, TAIL_BF16, TAIL_Q8_0, TAIL_F16 = 0, 1, 2, 3
LAYOUT_TILES, LAYOUT_ROWS = 0, 1
REGION = {"k_body": 0, "v_body": 1, "k_ring": 2, "v_ring": 3, "sigma": 4, "slab": 5, "index": 6}
MAX_BATCH = 64

_FIELDS = ("n_layers", "max_seqs", "capacity", "n_q_heads", "n_kv_heads", "head_dim", "k_bits", "v_bits",
           "kvarn", "tail_len", "tail_slack", "tail_dtype", "layout", "index_dim", "index_pool", "k_min", "v_min",
           "k_axis")

SYMBOLS = ("kvq_config_validate", "kvq_cache_bytes", "kvq_region", "kvq_cache_init", "kvq_cache_destroy",
           "kvq_seq_reset", "kvq_seq_truncate", "kvq_seq_lengths", "kvq_workspace_bytes", "kvq_append", "kvq_tail_evict",
           "kvq_append_evict", "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_decode_attn_multi", "kvq_decode_step", "kvq_sparse_decode_attn", "kvq_sparse_decode_step", "kvq_index_write", "kvq_index_workspace_bytes", "kvq_index_select", "kvq_prefill_attn", "kvq_prefill_workspace_bytes", "kvq_timing_enable", "kvq_timing_read", "kvq_last_error")
KERNEL = {"decode": 0, "gather": 1, "combine": 2, "append": 3, "evict": 4, "append_evict": 5, "index": 6, "mq": 7}


_OPTIONAL = ("layout", "index_dim", "index_pool", "k_min", "v_min",
           "k_axis")


class Config(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in _FIELDS]


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvq error {status}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"kvq HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    CP = ctypes.POINTER(Config)
    IP = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "kvq_config_validate": (I32, [CP]),
        "kvq_cache_bytes": (SZ, [CP]),
        "kvq_region": (I32, [CP, I32, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
        "kvq_cache_init": (I32, [CP, P, SZ, P, ctypes.POINTER(P)]),
        "kvq_cache_destroy": (None, [P]),
        "kvq_seq_reset": (I32, [P, I32, I32, IP, P]),
        "kvq_seq_truncate": (I32, [P, I32, I32, IP, IP]),
        "kvq_seq_lengths": (I32, [P, I32, I32, IP, IP]),
        "kvq_workspace_bytes": (SZ, [P, I32, I32]),
        "kvq_append": (I32, [P, I32, I32, IP, IP, P, P, P]),
        "kvq_append_evict": (I32, [P, I32, I32, IP, IP, P, P, P]),
        "kvq_decode_step": (I32, [P, I32, I32, IP, P, P, P, P, F, P, SZ, P]),
        "kvq_tail_evict": (I32, [P, I32, I32, IP, P]),
        "kvq_decode_attn": (I32, [P, I32, I32, IP, P, P, F, P, SZ, P]),
        "kvq_decode_attn_noalloc": (I32, [P, I32, I32, IP, P, P, F, P]),
        "kvq_decode_attn_multi": (I32, [P, I32, I32, IP, I32, P, P, F, P, SZ, P]),
        "kvq_sparse_decode_attn": (I32, [P, I32, I32, IP, P, P, I32, P, F, P, SZ, P]),
        "kvq_sparse_decode_step": (I32, [P, I32, I32, IP, P, P, P, P, I32, P, F, P, SZ, P]),
        "kvq_index_write": (I32, [P, I32, I32, IP, IP, P, P]),
        "kvq_prefill_attn": (I32, [P, I32, I32, IP, IP, P, P, P, P, F, P, SZ, P]),
        "kvq_prefill_workspace_bytes": (SZ, [P, I32, I32, I32]),
        "kvq_index_workspace_bytes": (SZ, [P, I32, I32]),
        "kvq_index_select": (I32, [P, I32, I32, IP, P, I32, I32, P, P, SZ, P]),
        "kvq_timing_enable": (I32, [P, I32]),
        "kvq_timing_read": (I32, [P, I32, ctypes.POINTER(ctypes.c_double), IP]),
        "kvq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, _lib.kvq_last_error().decode())


def make_config(cfg: Dict[str, int]) -> Config:
    """kvq_config from a dict; "layout" defaults to LAYOUT_TILES, "index_dim" / "index_pool" to 0 (no indexer)."""
    return Config(*[int(cfg.get(f, 0) if f in _OPTIONAL else cfg[f]) for f in _FIELDS])


def config_validate(cfg: Dict[str, int]) -> None:
    c = make_config(cfg)
    _check(_lib.kvq_config_validate(ctypes.byref(c)))


def cache_bytes(cfg: Dict[str, int]) -> int:
    c = make_config(cfg)
    return int(_lib.kvq_cache_bytes(ctypes.byref(c)))


def region(cfg: Dict[str, int], layer: int, seq: int, name: str):
    c = make_config(cfg)
    off, size = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.kvq_region(ctypes.byref(c), layer, seq, REGION[name], ctypes.byref(off), ctypes.byref(size)))
    return off.value, size.value


def _ids(seq_ids: Sequence[int]):
    arr = (ctypes.c_int32 * len(seq_ids))(*[int(s) for s in seq_ids])
    return arr


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Cache:
    """A quantized KV cache over a torch-allocated device arena (the arena is owned by this object)."""

    def __init__(self, cfg: Dict[str, int], arena: Optional[torch.Tensor] = None, stream=None):
        self.cfg = dict(cfg)
        self._c = make_config(self.cfg)
        nbytes = cache_bytes(self.cfg)
        if nbytes == 0:
            config_validate(self.cfg)
        if arena is None:
            arena = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.arena = arena
        h = ctypes.c_void_p()
        _check(_lib.kvq_cache_init(ctypes.byref(self._c), _dev(arena, torch.uint8, "arena"), arena.numel(),
                                   ctypes.c_void_p(_stream(stream)), ctypes.byref(h)))
        self._h = h
        self.hq = self.cfg["n_q_heads"]
        self.hk = self.cfg["n_kv_heads"]
        self.d = self.cfg["head_dim"]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _lib.kvq_cache_destroy(h)
            self._h = None

    # ---------------------------------------------------------------- state
    def lengths(self, layer: int, seq: int):
        ln, bl = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.kvq_seq_lengths(self._h, layer, seq, ctypes.byref(ln), ctypes.byref(bl)))
        return ln.value, bl.value

    def seq_reset(self, layer: int, seq_ids: Sequence[int], stream=None):
        _check(_lib.kvq_seq_reset(self._h, layer, len(seq_ids), _ids(seq_ids), ctypes.c_void_p(_stream(stream))))

    def seq_truncate(self, layer: int, seq_ids: Sequence[int], new_lens: Sequence[int]):
        """Drop the newest positions (still in the ring) of each sequence down to new_lens[i]."""
        if len(new_lens) != len(seq_ids):
            raise ValueError("one new length per sequence")
        _check(_lib.kvq_seq_truncate(self._h, layer, len(seq_ids), _ids(seq_ids), _ids(new_lens)))

    def workspace_bytes(self, n_seqs: int, max_len: int) -> int:
        return int(_lib.kvq_workspace_bytes(self._h, n_seqs, max_len))

    def workspace(self, n_seqs: int, max_len: int) -> torch.Tensor:
        """A workspace for n_seqs sequences of up to max_len positions (kept by the cache and grown on
        demand, so repeated calls return the same memory)."""
        n = max(self.workspace_bytes(n_seqs, max_len), 256)
        ws = getattr(self, "_ws", None)
        if ws is None or ws.numel() < n:
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            self._ws = ws
        return ws

    # ---------------------------------------------------------------- launch timing
    def timing(self, enable: bool = True):
        """Bracket every launch of this cache with HIP events on its stream (drops earlier records)."""
        _check(_lib.kvq_timing_enable(self._h, 1 if enable else 0))

    def timing_read(self, kernel: str):
        """(total ms, launches) recorded for a kernel kind: decode, gather, combine, append, evict."""
        ms, n = ctypes.c_double(), ctypes.c_int32()
        _check(_lib.kvq_timing_read(self._h, KERNEL[kernel], ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    # ---------------------------------------------------------------- the calls
    def append(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], k: torch.Tensor,
               v: torch.Tensor, stream=None):
        """k, v: bf16 (or int16/uint16 bit patterns) [sum(n_new), Hkv, D] on the device."""
        self._append(_lib.kvq_append, layer, seq_ids, n_new, k, v, stream)

    def append_evict(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], k: torch.Tensor,
                     v: torch.Tensor, stream=None):
        """append() then tail_evict() on the same sequences (one kernel launch for a decode step)."""
        self._append(_lib.kvq_append_evict, layer, seq_ids, n_new, k, v, stream)

    def _append(self, fn, layer, seq_ids, n_new, k, v, stream):
        total = int(sum(int(n) for n in n_new))
        for name, t in (("k", k), ("v", v)):
            if t.numel() != total * self.hk * self.d:
                raise ValueError(f"{name} has {t.numel()} elements, expected {total * self.hk * self.d}")
        kp = _dev(k, k.dtype, "k") if total else ctypes.c_void_p(0)
        vp = _dev(v, v.dtype, "v") if total else ctypes.c_void_p(0)
        if total and k.element_size() != 2:
            raise ValueError("k/v must hold 16-bit bf16 values")
        nn = (ctypes.c_int32 * len(n_new))(*[int(n) for n in n_new])
        _check(fn(self._h, layer, len(seq_ids), _ids(seq_ids), nn, kp, vp, ctypes.c_void_p(_stream(stream))))

    def tail_evict(self, layer: int, seq_ids: Sequence[int], stream=None):
        _check(_lib.kvq_tail_evict(self._h, layer, len(seq_ids), _ids(seq_ids), ctypes.c_void_p(_stream(stream))))

    def decode_attn(self, layer: int, seq_ids: Sequence[int], q: torch.Tensor, out: Optional[torch.Tensor] = None,
                    softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None):
        n = len(seq_ids)
        if q.numel() != n * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, Hq, D]")
        if out is None:
            out = torch.empty((n, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            max_len = max(self.lengths(layer, s)[0] for s in seq_ids)
            workspace = self.workspace(n, max(1, max_len))
        _check(_lib.kvq_decode_attn(self._h, layer, n, _ids(seq_ids), _dev(q, q.dtype, "q"),
                                    _dev(out, torch.float32, "out"), float(softmax_scale),
                                    _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                    ctypes.c_void_p(_stream(stream))))
        return out

    def decode_attn_noalloc(self, layer: int, seq_ids: Sequence[int], q: torch.Tensor, out: torch.Tensor,
                            softmax_scale: float = 0.0, stream=None):
        """decode_attn() with the split partials in the library's static scratch (no workspace): for callers that
        cannot allocate. out must be given (fp32 [n_seqs, Hq, D]); calls on one GPU must not overlap."""
        n = len(seq_ids)
        if q.numel() != n * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, Hq, D]")
        if out.numel() != n * self.hq * self.d:
            raise ValueError("out must be fp32 [n_seqs, Hq, D]")
        _check(_lib.kvq_decode_attn_noalloc(self._h, layer, n, _ids(seq_ids), _dev(q, q.dtype, "q"),
                                            _dev(out, torch.float32, "out"), float(softmax_scale),
                                            ctypes.c_void_p(_stream(stream))))
        return out

    def decode_attn_multi(self, layer: int, seq_ids: Sequence[int], q: torch.Tensor, out: Optional[torch.Tensor] = None,
                          softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None):
        """Decode of the last T cached positions of each sequence at once, causal among them (verification of
        drafted tokens). q: bf16 [n_seqs, T, Hq, D]; returns fp32 [n_seqs, T, Hq, D]."""
        n = len(seq_ids)
        if q.dim() != 4 or q.shape[0] != n or q.shape[2] != self.hq or q.shape[3] != self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, T, Hq, D]")
        t = q.shape[1]
        if out is None:
            out = torch.empty((n, t, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            max_len = max(self.lengths(layer, s)[0] for s in seq_ids)
            workspace = self.workspace(max(1, min(n * t, KVQ_MAX_BATCH)), max(1, max_len))
        _check(_lib.kvq_decode_attn_multi(self._h, layer, n, _ids(seq_ids), t, _dev(q, q.dtype, "q"),
                                          _dev(out, torch.float32, "out"), float(softmax_scale),
                                          _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                          ctypes.c_void_p(_stream(stream))))
        return out

    def decode_step(self, layer: int, seq_ids: Sequence[int], k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                    out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                    workspace: Optional[torch.Tensor] = None, stream=None):
        """append_evict() of one token per sequence, then decode_attn() (one launch for a decode step).
        k, v: bf16 [n_seqs, Hkv, D]; q: bf16 [n_seqs, Hq, D]."""
        n = len(seq_ids)
        for name, t in (("k", k), ("v", v)):
            if t.numel() != n * self.hk * self.d or t.element_size() != 2:
                raise ValueError(f"{name} must be bf16 [n_seqs, Hkv, D]")
        if q.numel() != n * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, Hq, D]")
        if out is None:
            out = torch.empty((n, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            max_len = max(self.lengths(layer, s)[0] for s in seq_ids) + 1
            workspace = self.workspace(n, max_len)
        _check(_lib.kvq_decode_step(self._h, layer, n, _ids(seq_ids), _dev(k, k.dtype, "k"), _dev(v, v.dtype, "v"),
                                    _dev(q, q.dtype, "q"), _dev(out, torch.float32, "out"), float(softmax_scale),
                                    _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                    ctypes.c_void_p(_stream(stream))))
        return out

    def sparse_decode_attn(self, layer: int, seq_ids: Sequence[int], q: torch.Tensor, positions: torch.Tensor,
                           out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                           workspace: Optional[torch.Tensor] = None, stream=None):
        n = len(seq_ids)
        if q.numel() != n * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, Hq, D]")
        if positions.dim() != 2 or positions.shape[0] != n:
            raise ValueError("positions must be int32 [n_seqs, budget]")
        budget = positions.shape[1]
        if out is None:
            out = torch.empty((n, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(n, budget)
        _check(_lib.kvq_sparse_decode_attn(self._h, layer, n, _ids(seq_ids), _dev(q, q.dtype, "q"),
                                           _dev(positions, torch.int32, "positions"), budget,
                                           _dev(out, torch.float32, "out"), float(softmax_scale),
                                           _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                           ctypes.c_void_p(_stream(stream))))
        return out

    def sparse_decode_step(self, layer: int, seq_ids: Sequence[int], k: torch.Tensor, v: torch.Tensor,
                           q: torch.Tensor, positions: torch.Tensor, out: Optional[torch.Tensor] = None,
                           softmax_scale: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None):
        """append() of one token per sequence, then sparse_decode_attn() (one launch without a tail ring).
        k, v: bf16 [n_seqs, Hkv, D]; q: bf16 [n_seqs, Hq, D]; positions: int32 [n_seqs, budget] (after the
        append: the new token is at the old length)."""
        n = len(seq_ids)
        for name, t in (("k", k), ("v", v)):
            if t.numel() != n * self.hk * self.d or t.element_size() != 2:
                raise ValueError(f"{name} must be bf16 [n_seqs, Hkv, D]")
        if q.numel() != n * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [n_seqs, Hq, D]")
        if positions.dim() != 2 or positions.shape[0] != n:
            raise ValueError("positions must be int32 [n_seqs, budget]")
        budget = positions.shape[1]
        if out is None:
            out = torch.empty((n, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(n, budget)
        _check(_lib.kvq_sparse_decode_step(self._h, layer, n, _ids(seq_ids), _dev(k, k.dtype, "k"),
                                           _dev(v, v.dtype, "v"), _dev(q, q.dtype, "q"),
                                           _dev(positions, torch.int32, "positions"), budget,
                                           _dev(out, torch.float32, "out"), float(softmax_scale),
                                           _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                           ctypes.c_void_p(_stream(stream))))
        return out

    # ---------------------------------------------------------------- the QSA indexer
    def index_write(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], keys: torch.Tensor, stream=None):
        """Pool and store the indexer keys of the newest n_new[i] positions of each sequence (after append()).
        keys: bf16 (or 16-bit bit patterns) [sum(n_new), index_dim] on the device."""
        total = int(sum(int(n) for n in n_new))
        dim = self.cfg.get("index_dim", 0)
        if total and dim and (keys.numel() != total * dim or keys.element_size() != 2):
            raise ValueError(f"keys must be 16-bit [{total}, {dim}]")   # (a cache without an indexer: the library says so)
        kp = _dev(keys, keys.dtype, "keys") if total else ctypes.c_void_p(0)
        nn = (ctypes.c_int32 * len(n_new))(*[int(n) for n in n_new])
        _check(_lib.kvq_index_write(self._h, layer, len(seq_ids), _ids(seq_ids), nn, kp,
                                    ctypes.c_void_p(_stream(stream))))

    def index_workspace_bytes(self, n_seqs: int, max_len: int) -> int:
        return int(_lib.kvq_index_workspace_bytes(self._h, n_seqs, max_len))

    def index_select(self, layer: int, seq_ids: Sequence[int], query: torch.Tensor, budget: int, n_recent: int = 0,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
        """Positions chosen by the indexer: int32 [n_seqs, budget] (ascending, -1 padded). query: bf16 [n_seqs, 32]."""
        n = len(seq_ids)
        if query.numel() != n * 32 or query.element_size() != 2:
            raise ValueError("query must be bf16 [n_seqs, 32]")
        if out is None:
            out = torch.empty((n, budget), dtype=torch.int32, device=query.device)
        if workspace is None:
            max_len = max(self.lengths(layer, s)[0] for s in seq_ids)
            need = max(self.index_workspace_bytes(n, max_len), 256)
            ws = getattr(self, "_iws", None)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                self._iws = ws
            workspace = ws
        _check(_lib.kvq_index_select(self._h, layer, n, _ids(seq_ids), _dev(query, query.dtype, "query"), int(budget),
                                     int(n_recent), _dev(out, torch.int32, "out"),
                                     _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                     ctypes.c_void_p(_stream(stream))))
        return out

    # ---------------------------------------------------------------- chunked prefill
    def prefill_workspace_bytes(self, n_seqs: int, max_new: int, max_len: int) -> int:
        return int(_lib.kvq_prefill_workspace_bytes(self._h, n_seqs, max_new, max_len))

    def prefill_attn(self, layer: int, seq_ids: Sequence[int], n_new: Sequence[int], k: torch.Tensor, v: torch.Tensor,
                     q: torch.Tensor, out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                     workspace: Optional[torch.Tensor] = None, stream=None):
        """append() of n_new[i] tokens per sequence, then causal attention of their queries over the cache as it
        then stands. k, v: bf16 [sum(n_new), Hkv, D]; q: bf16 [sum(n_new), Hq, D]; returns fp32 [sum(n_new), Hq, D]."""
        total = int(sum(int(n) for n in n_new))
        for name, t in (("k", k), ("v", v)):
            if t.numel() != total * self.hk * self.d or t.element_size() != 2:
                raise ValueError(f"{name} must be bf16 [{total}, Hkv, D]")
        if q.numel() != total * self.hq * self.d or q.element_size() != 2:
            raise ValueError("q must be bf16 [sum(n_new), Hq, D]")
        if out is None:
            out = torch.empty((total, self.hq, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            max_new = max(1, max(int(x) for x in n_new))
            max_len = max(1, max(self.lengths(layer, s)[0] + int(x) for s, x in zip(seq_ids, n_new)))
            need = max(self.prefill_workspace_bytes(len(seq_ids), max_new, max_len), 256)
            ws = getattr(self, "_pws", None)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                self._pws = ws
            workspace = ws
        if total == 0:
            return out
        nn = (ctypes.c_int32 * len(n_new))(*[int(x) for x in n_new])
        _check(_lib.kvq_prefill_attn(self._h, layer, len(seq_ids), _ids(seq_ids), nn, _dev(k, k.dtype, "k"),
                                     _dev(v, v.dtype, "v"), _dev(q, q.dtype, "q"), _dev(out, torch.float32, "out"),
                                     float(softmax_scale), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                     ctypes.c_void_p(_stream(stream))))
        return out
