"""Cache state machine: qN_0 or qN_1 body, precision tail / 8-bit ring, requantization (oracle).

Test infrastructure only. Follows, step by step:

* qN_0 body with separate K and V widths (KVarN benchmark page, K/V pair table;
  "Hard numbers on Qwen3.8-27B's KV cache" page, K 6-bit / V 5-bit setting D); either
  side may instead be qN_1, a scale and a minimum per block (BeeLlama.cpp v0.4.1 page,
  q2_1 .. q6_1; KVarN benchmark page, the q8_0-q5_1 pair). The 8-bit ring stays q8_0.
* Precision tail: the newest W tokens are kept in bf16 or f16, the rest quantized as
  usual (BeeLlama.cpp v0.4.1 page, KV cache precision tail paragraph and feature list).
  Reading for f16: the bf16 input is converted to IEEE binary16 with round to nearest
  even (exact for every bf16 value of magnitude in [2^-14, 65504]; smaller ones round to
  f16 subnormals, larger ones overflow to infinity).
* 8-bit recent ring: the newest 2,048 positions sit in an 8-bit ring; below the
  window the output equals a q8_0 cache (Qwen3.8-27B page, KV low-bit section).
  Reading: ring rows are q8_0 blocks; eviction requantizes the dequantized q8_0
  values (double quantization).
* Token-axis K (Qwen3.8-27B page, reader comment on KIVI-style per-channel K): a K
  block is the 32 positions of one channel in a position tile. Reading: such a block
  can only be quantized once all its positions are known, so the body grows by whole
  tiles: tokens leave the ring a tile at a time (the ring holds the window plus the
  tile still filling, so it needs at least 32 slots of slack), and tail_evict keeps
  between W and W + 31 positions in the ring. V stays per token.
* Tokens leaving the window are requantized into the low-bit body; this needs two
  KV paths per layer and per-position branching (Qwen3.8-27B page, reader comment
  on the window boundary).
* KVarN (BeeLlama.cpp v0.4.1 page, KVarN paragraph): per-channel sigma from the
  first appended chunk, applied to every row before block quantization.

Readings: the ring holds R = W + S slots (S = slack, 512 by default, which makes
the KV MiB table's tail rows exact); position p lives in slot p mod R. ``append``
evicts the oldest ring rows only when the ring would overflow; tokens that are
already behind the window after an append go to the body through the ring
representation, so the body never depends on chunking. ``tail_evict`` drains the
ring to the newest W. A decode step appends into the slack, then evicts.
"""
from __future__ import annotations

import numpy as np

from .layout import (pack_k_rows, pack_k_tiles, pack_k_tiles_token_axis, pack_bf16_k_tiles, pack_v_tiles,
                     pack_bf16_v_tiles, slab_layout, TILE)
from .quant import quantize_blocks, quantize_blocks_min, kvarn_sigma, normalize, dequantize_blocks, dequantize_blocks_min
from . import indexer

TAIL_NONE, TAIL_BF16, TAIL_Q8, TAIL_F16 = 0, 1, 2, 3
_TAIL_16 = (TAIL_BF16, TAIL_F16)   # rings of 16-bit values
LAYOUT_TILES, LAYOUT_ROWS = 0, 1


def _bf16_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _f16_bits(x32):
    """IEEE binary16 bit patterns of fp32 values (round to nearest even)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


def _f16_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


class _SeqState:
    def __init__(self, cfg, lay):
        hk, d = cfg["n_kv_heads"], cfg["head_dim"]
        nb = d // 32
        cap32 = lay["cap32"]
        self.len = 0
        self.body_len = 0
        self.calibrated = False
        self.sigma = np.zeros((hk, 2, d), dtype=np.float16)
        self.ku = np.zeros((cap32, hk, d), dtype=np.uint8)
        self.kd = np.zeros((cap32, hk, nb), dtype=np.float16)
        self.vu = np.zeros((cap32, hk, d), dtype=np.uint8)
        self.vd = np.zeros((cap32, hk, nb), dtype=np.float16)
        # qN_1 bodies: the block minima (zero rows for a qN_0 side, never read)
        self.km = np.zeros((cap32, hk, nb), dtype=np.float16)
        self.vm = np.zeros((cap32, hk, nb), dtype=np.float16)
        # token-axis K: one scale (and minimum) per (position tile, KV head, channel)
        self.ktd = np.zeros((cap32 // 32, hk, d), dtype=np.float16)
        self.ktm = np.zeros((cap32 // 32, hk, d), dtype=np.float16)
        if cfg.get("index_dim", 0):
            self.ikey = np.zeros((cap32, indexer.POOLED), dtype=np.uint16)   # pooled index keys, bf16 bits
        r = lay["ring_slots"]
        if cfg["tail_len"] > 0 and cfg["tail_dtype"] in _TAIL_16:
            self.rk = np.zeros((r, hk, d), dtype=np.uint16)
            self.rv = np.zeros((r, hk, d), dtype=np.uint16)
        elif cfg["tail_len"] > 0:
            self.rku = np.zeros((r, hk, d), dtype=np.uint8)
            self.rkd = np.zeros((r, hk, nb), dtype=np.float16)
            self.rvu = np.zeros((r, hk, d), dtype=np.uint8)
            self.rvd = np.zeros((r, hk, nb), dtype=np.float16)


class OracleCache:
    """Mirror of the library's cache semantics on the CPU, one (layer, sequence) at a time."""

    def __init__(self, cfg: dict):
        self.cfg = dict(cfg)
        self.lay = slab_layout(self.cfg)
        self.W = cfg["tail_len"]
        self.R = self.lay["ring_slots"]
        self.tail = cfg["tail_dtype"] if self.W > 0 else TAIL_NONE
        self.rows = cfg.get("layout", LAYOUT_TILES) == LAYOUT_ROWS   # V stored as rows, like K
        self.k_min = bool(cfg.get("k_min", 0))   # qN_1 bodies (scale and minimum per block)
        self.v_min = bool(cfg.get("v_min", 0))
        self.k_tok = bool(cfg.get("k_axis", 0))  # token-axis K: blocks of 32 positions of one channel
        self.state = {}

    # ------------------------------------------------------------------ helpers
    def st(self, layer: int, seq: int) -> _SeqState:
        key = (layer, seq)
        if key not in self.state:
            self.state[key] = _SeqState(self.cfg, self.lay)
        return self.state[key]

    def _ring_value(self, s: _SeqState, slots) -> tuple:
        """fp32 ring representation r(x) of K and V at ring slots: [n, Hkv, D] each."""
        if self.tail == TAIL_BF16:
            return _bf16_f32(s.rk[slots]), _bf16_f32(s.rv[slots])
        if self.tail == TAIL_F16:
            return _f16_f32(s.rk[slots]), _f16_f32(s.rv[slots])
        k = dequantize_blocks(s.rku[slots], s.rkd[slots], 8).astype(np.float32)   # exact c * d16
        v = dequantize_blocks(s.rvu[slots], s.rvd[slots], 8).astype(np.float32)
        return k, v

    def _ring_rep_of_input(self, k_bits, v_bits) -> tuple:
        """r(x) for fresh inputs (what the ring would store, read back as fp32)."""
        k = _bf16_f32(k_bits)
        v = _bf16_f32(v_bits)
        if self.tail == TAIL_F16:
            k, v = _f16_f32(_f16_bits(k)), _f16_f32(_f16_bits(v))
        if self.tail == TAIL_Q8:
            ku, kd = quantize_blocks(k, 8)
            vu, vd = quantize_blocks(v, 8)
            k = dequantize_blocks(ku, kd, 8).astype(np.float32)
            v = dequantize_blocks(vu, vd, 8).astype(np.float32)
        return k, v

    def _write_body(self, s: _SeqState, pos: np.ndarray, k32, v32):
        """Quantize fp32 rows (after the ring representation) into body positions."""
        if len(pos) == 0:
            return
        if self.cfg["kvarn"]:
            k32 = normalize(k32, s.sigma[:, 0, :])
            v32 = normalize(v32, s.sigma[:, 1, :])
        if self.k_tok:
            # whole position tiles only: quantize each channel's 32 values of a tile as one block
            assert pos[0] % TILE == 0 and len(pos) % TILE == 0 and np.all(np.diff(pos) == 1)
            ntl = len(pos) // TILE
            hk, d = k32.shape[1], k32.shape[2]
            xt = np.ascontiguousarray(k32.reshape(ntl, TILE, hk, d).transpose(0, 2, 3, 1))   # [tile, head, ch, pos]
            tl = pos[::TILE] // TILE
            if self.k_min:
                u, d16, m16 = quantize_blocks_min(xt, self.cfg["k_bits"])
                s.ktm[tl] = m16[..., 0]
            else:
                u, d16 = quantize_blocks(xt, self.cfg["k_bits"])
            s.ktd[tl] = d16[..., 0]
            s.ku[pos] = u.transpose(0, 3, 1, 2).reshape(len(pos), hk, d)
        elif self.k_min:
            s.ku[pos], s.kd[pos], s.km[pos] = quantize_blocks_min(k32, self.cfg["k_bits"])
        else:
            s.ku[pos], s.kd[pos] = quantize_blocks(k32, self.cfg["k_bits"])
        if self.v_min:
            s.vu[pos], s.vd[pos], s.vm[pos] = quantize_blocks_min(v32, self.cfg["v_bits"])
        else:
            s.vu[pos], s.vd[pos] = quantize_blocks(v32, self.cfg["v_bits"])

    def _write_ring(self, s: _SeqState, pos: np.ndarray, k_bits, v_bits):
        if len(pos) == 0:
            return
        slots = pos % self.R
        if self.tail == TAIL_BF16:
            s.rk[slots] = k_bits
            s.rv[slots] = v_bits
        elif self.tail == TAIL_F16:
            s.rk[slots] = _f16_bits(_bf16_f32(k_bits))
            s.rv[slots] = _f16_bits(_bf16_f32(v_bits))
        else:
            s.rku[slots], s.rkd[slots] = quantize_blocks(_bf16_f32(k_bits), 8)
            s.rvu[slots], s.rvd[slots] = quantize_blocks(_bf16_f32(v_bits), 8)

    def _evict_to(self, s: _SeqState, target: int):
        """Requantize ring positions [body_len, target) into the body."""
        if target <= s.body_len:
            return
        pos = np.arange(s.body_len, target)
        k32, v32 = self._ring_value(s, pos % self.R)
        self._write_body(s, pos, k32, v32)
        s.body_len = target

    # ------------------------------------------------------------------ the calls
    def append(self, layer: int, seq_ids, n_new, k_bits: np.ndarray, v_bits: np.ndarray):
        """k_bits, v_bits: bf16 bit patterns [sum(n_new), Hkv, D], sequences in order."""
        off = 0
        for sid, n in zip(seq_ids, n_new):
            n = int(n)
            kb = k_bits[off:off + n]
            vb = v_bits[off:off + n]
            off += n
            s = self.st(layer, sid)
            if s.len + n > self.cfg["capacity"]:
                raise ValueError("capacity")
            if n == 0:
                continue
            if self.cfg["kvarn"] and not s.calibrated:
                sig_k = kvarn_sigma(_bf16_f32(kb))            # [Hkv, D]
                sig_v = kvarn_sigma(_bf16_f32(vb))
                s.sigma = np.stack([sig_k, sig_v], axis=1)
                s.calibrated = True
            new_len = s.len + n
            pos = np.arange(s.len, new_len)
            if self.tail == TAIL_NONE:
                self._write_body(s, pos, _bf16_f32(kb), _bf16_f32(vb))
                s.len = s.body_len = new_len
                continue
            new_body = max(s.body_len, new_len - self.R)
            if self.k_tok:
                # the body grows by whole tiles: positions of a tile leave the ring together, ring rows and new
                # tokens behind the window in one write
                new_body = max(s.body_len, -(-(new_len - self.R) // TILE) * TILE)
                if new_body > s.body_len:
                    p_all = np.arange(s.body_len, new_body)
                    old_p = p_all[p_all < s.len]
                    new_p = p_all[p_all >= s.len]
                    k_old, v_old = self._ring_value(s, old_p % self.R)
                    k_new, v_new = self._ring_rep_of_input(kb[new_p - s.len], vb[new_p - s.len])
                    self._write_body(s, p_all, np.concatenate([k_old, k_new]), np.concatenate([v_old, v_new]))
                keep = pos[pos >= new_body]
                self._write_ring(s, keep, kb[keep - s.len], vb[keep - s.len])
                s.len = new_len
                s.body_len = new_body
                continue
            # oldest ring rows leave first (only when the ring would overflow)
            self._evict_to(s, min(new_body, s.len))
            # new tokens already behind the window: through the ring representation
            direct = pos[pos < new_body]
            if len(direct):
                sel = direct - s.len
                k32, v32 = self._ring_rep_of_input(kb[sel], vb[sel])
                self._write_body(s, direct, k32, v32)
            keep = pos[pos >= new_body]
            self._write_ring(s, keep, kb[keep - s.len], vb[keep - s.len])
            s.len = new_len
            s.body_len = new_body

    def tail_evict(self, layer: int, seq_ids):
        for sid in seq_ids:
            s = self.st(layer, sid)
            if self.tail == TAIL_NONE:
                continue
            target = s.len - self.W
            if self.k_tok:   # whole tiles only
                target = target // TILE * TILE
            self._evict_to(s, max(s.body_len, target))

    def truncate(self, layer: int, seq_ids, new_lens):
        """Drop the newest positions of each sequence down to new_lens[i], which must lie in [body_len, len]: only
        rows still in the ring can be dropped (drafted tokens a verification step rejected; Qwen3.8-27B page,
        decode-speed paragraph on MTP drafting). The dropped ring rows stay in their slots until later appends
        write those slots again; KVarN calibration is kept."""
        for sid, n in zip(seq_ids, new_lens):
            s = self.st(layer, sid)
            if not s.body_len <= int(n) <= s.len:
                raise ValueError(f"truncate to {n} outside [body_len {s.body_len}, len {s.len}]")
            s.len = int(n)

    # ------------------------------------------------------------------ the indexer (offload page, QSA)
    def index_write(self, layer: int, seq_ids, n_new, key_bits: np.ndarray):
        """Pool and store the indexer keys of the newest n_new[i] positions of each sequence (already appended):
        key_bits bf16 [sum(n_new), index_dim], sequences in order."""
        ratio = self.cfg["index_pool"]
        off = 0
        for sid, n in zip(seq_ids, n_new):
            n = int(n)
            s = self.st(layer, sid)
            if n > s.len:
                raise ValueError(f"sequence {sid} holds {s.len} positions, fewer than {n} keys")
            if n:
                s.ikey[s.len - n:s.len] = indexer.pool_keys(key_bits[off:off + n], ratio)
            off += n

    def index_select(self, layer: int, seq_ids, query_bits: np.ndarray, budget: int, n_recent: int = 0):
        """Positions chosen by the indexer for each sequence: int32 [n_seqs, budget] (ascending, -1 padded)."""
        out = []
        for i, sid in enumerate(seq_ids):
            s = self.st(layer, sid)
            m = max(s.len - n_recent, 0)
            sc = indexer.scores(query_bits[i], s.ikey[:m])
            out.append(indexer.select(sc, s.len, budget, n_recent))
        return np.stack(out)

    # ------------------------------------------------------------------ reading
    def lengths(self, layer: int, seq: int):
        s = self.st(layer, seq)
        return s.len, s.body_len

    def dequantized(self, layer: int, seq: int, positions=None):
        """Exact fp64 K^, V^ [n, Hkv, D] at positions (default: all of [0, len))."""
        s = self.st(layer, seq)
        if positions is None:
            positions = np.arange(s.len)
        positions = np.asarray(positions, dtype=np.int64)
        d = self.cfg["head_dim"]
        hk = self.cfg["n_kv_heads"]
        k = np.zeros((len(positions), hk, d))
        v = np.zeros((len(positions), hk, d))
        in_body = positions < s.body_len
        pb = positions[in_body]
        if len(pb):
            if self.k_tok:
                tl = pb // TILE
                c = s.ku[pb].astype(np.float64)
                if self.k_min:
                    kb = c * s.ktd[tl].astype(np.float64) + s.ktm[tl].astype(np.float64)
                else:
                    kb = (c - (1 << (self.cfg["k_bits"] - 1))) * s.ktd[tl].astype(np.float64)
            else:
                kb = (dequantize_blocks_min(s.ku[pb], s.kd[pb], s.km[pb]) if self.k_min
                      else dequantize_blocks(s.ku[pb], s.kd[pb], self.cfg["k_bits"]))
            vb = (dequantize_blocks_min(s.vu[pb], s.vd[pb], s.vm[pb]) if self.v_min
                  else dequantize_blocks(s.vu[pb], s.vd[pb], self.cfg["v_bits"]))
            if self.cfg["kvarn"]:
                kb = kb * s.sigma[:, 0, :].astype(np.float64)
                vb = vb * s.sigma[:, 1, :].astype(np.float64)
            k[in_body], v[in_body] = kb, vb
        pr = positions[~in_body]
        if len(pr):
            kr, vr = self._ring_value(s, pr % self.R)
            k[~in_body], v[~in_body] = kr.astype(np.float64), vr.astype(np.float64)
        return k, v

    # ------------------------------------------------------------------ bytes
    def region_bytes(self, layer: int, seq: int, region: str, head: int, lo: int, hi: int) -> np.ndarray:
        """Packed bytes of one head's region for positions / slots [lo, hi).

        Tile layout: tiles lo//32 .. hi//32 - 1 (lo, hi multiples of 32) of every region;
        row layout: rows lo..hi-1. sigma: the [2, D] fp16 block of the head."""
        s = self.st(layer, seq)
        kb, vb = self.cfg["k_bits"], self.cfg["v_bits"]
        d = self.cfg["head_dim"]
        km = s.km[lo:hi, head] if self.k_min else None
        vm = s.vm[lo:hi, head] if self.v_min else None
        if region == "k_body" and not self.rows and self.k_tok:
            assert lo % TILE == 0 and hi % TILE == 0
            return pack_k_tiles_token_axis(s.ku[lo:hi, head].reshape(-1, TILE, d), s.ktd[lo // TILE:hi // TILE, head], kb,
                                           s.ktm[lo // TILE:hi // TILE, head] if self.k_min else None)
        if region == "k_body" and not self.rows:
            assert lo % TILE == 0 and hi % TILE == 0
            return pack_k_tiles(s.ku[lo:hi, head].reshape(-1, TILE, d), s.kd[lo:hi, head].reshape(-1, TILE, d // 32), kb,
                                None if km is None else km.reshape(-1, TILE, d // 32))
        if region == "k_ring" and not self.rows:
            assert lo % TILE == 0 and hi % TILE == 0
            if self.tail in _TAIL_16:   # 16-bit values, packed alike
                return pack_bf16_k_tiles(s.rk[lo:hi, head].reshape(-1, TILE, d))
            return pack_k_tiles(s.rku[lo:hi, head].reshape(-1, TILE, d), s.rkd[lo:hi, head].reshape(-1, TILE, d // 32), 8)
        if region == "k_body":
            return pack_k_rows(s.ku[lo:hi, head], s.kd[lo:hi, head], kb, km)
        if region == "v_body" and self.rows:
            return pack_k_rows(s.vu[lo:hi, head], s.vd[lo:hi, head], vb, vm)
        if region == "v_ring" and self.rows:
            if self.tail in _TAIL_16:   # 16-bit values, packed alike
                return np.ascontiguousarray(s.rv[lo:hi, head]).view(np.uint8)
            return pack_k_rows(s.rvu[lo:hi, head], s.rvd[lo:hi, head], 8)
        if region == "v_body":
            assert lo % TILE == 0 and hi % TILE == 0
            u = s.vu[lo:hi, head].reshape(-1, TILE, self.cfg["head_dim"])
            d = s.vd[lo:hi, head].reshape(-1, TILE, self.cfg["head_dim"] // 32)
            return pack_v_tiles(u, d, vb, None if vm is None else vm.reshape(-1, TILE, self.cfg["head_dim"] // 32))
        if region == "k_ring":
            if self.tail in _TAIL_16:   # 16-bit values, packed alike
                return np.ascontiguousarray(s.rk[lo:hi, head]).view(np.uint8)
            return pack_k_rows(s.rku[lo:hi, head], s.rkd[lo:hi, head], 8)
        if region == "v_ring":
            assert lo % TILE == 0 and hi % TILE == 0
            if self.tail in _TAIL_16:   # 16-bit values, packed alike
                return pack_bf16_v_tiles(s.rv[lo:hi, head].reshape(-1, TILE, self.cfg["head_dim"]))
            u = s.rvu[lo:hi, head].reshape(-1, TILE, self.cfg["head_dim"])
            d = s.rvd[lo:hi, head].reshape(-1, TILE, self.cfg["head_dim"] // 32)
            return pack_v_tiles(u, d, 8)
        if region == "sigma":
            return np.ascontiguousarray(s.sigma[head]).view(np.uint8).reshape(-1)
        if region == "index":
            return np.ascontiguousarray(s.ikey[lo:hi]).view(np.uint8).reshape(-1)
        raise ValueError(region)

    def slab_image(self, layer: int, seq: int) -> np.ndarray:
        """The whole packed slab of one (layer, sequence), as the arena should hold it."""
        lay = self.lay
        img = np.zeros(lay["slab"], dtype=np.uint8)
        hk = self.cfg["n_kv_heads"]
        cap32 = lay["cap32"]
        if self.rows:
            # position-major: [position][head][K row, V row] in the body and in the ring region
            for kreg, vreg, region, n in (("k_body", "v_body", "k_body", cap32), ("k_ring", "v_ring", "k_ring", self.R)):
                off, size = lay[region]
                if size == 0:
                    continue
                runs = np.stack([np.concatenate([self.region_bytes(layer, seq, kreg, h, 0, n).reshape(n, -1),
                                                 self.region_bytes(layer, seq, vreg, h, 0, n).reshape(n, -1)], axis=1)
                                 for h in range(hk)], axis=1)            # [n, head, K row + V row]
                img[off:off + size] = runs.reshape(-1)
            regions = ()
        else:
            regions = (("k_body", cap32), ("v_body", cap32), ("k_ring", self.R), ("v_ring", self.R))
        for region, n in regions:
            off, size = lay[region]
            if size == 0:
                continue
            per = size // hk
            for h in range(hk):
                img[off + h * per: off + (h + 1) * per] = self.region_bytes(layer, seq, region, h, 0, n).reshape(-1)
        off, size = lay["sigma"]
        if size:
            per = size // hk
            for h in range(hk):
                img[off + h * per: off + (h + 1) * per] = self.region_bytes(layer, seq, "sigma", h, 0, 0)
        off, size = lay["index"]
        if size:
            img[off:off + size] = self.region_bytes(layer, seq, "index", 0, 0, cap32)
        return img
