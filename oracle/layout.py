"""Byte layout of the cache arena and its exact size (oracle; test infrastructure only).

The pages fix only the *size* of a qN_0 block: N bits per value plus one fp16
scale per 32 values (BeeLlama.cpp v0.4.1 page, KV MiB table: q4_0 / q5_0 /
q6_0 / q8_0 at tail 0 = 1152 / 1408 / 1664 / 2176 MiB; KVarN benchmark page,
cache-size column). Where the bits go inside the arena is a design choice made
for the GPU consumer; this module is its plain, independent statement.

Code planes. An N-bit biased code u is split into bit planes of width w:
    N=2: [2]   N=3: [2, 1]   N=4: [4]   N=5: [4, 1]   N=6: [4, 2]
    N=7: [4, 2, 1]   N=8: [8]
taken from the least significant bits upward (u = sum_k plane_k << shift_k).

Pieces. A piece is 8 codes e_0..e_7 of one plane. For w in {1, 2, 4}, 4/w pieces
share a little-endian 32-bit word; element i of piece p sits at bit
16*(i % 2) + 4*w*p + w*(i // 2). For w = 8 a piece is 8 bytes, e_i in byte i.

K rows (body, and the q8_0 ring): one row per (position, KV head). For lane
group j in 0..3 and block b, piece (j, b) holds channels 32*b + 8*j + i. A row is,
for each plane: for j = 0..3 the pieces b = 0..NB-1; then the NB fp16 block
scales in block order. Row bytes = NB * (4N + 2).

K tiles (tile layout; body and q8_0 ring): the K rows of 32 consecutive positions of
one KV head, rearranged so that a wave reads them with 1 KiB contiguous loads. For
subtile s in 0..1 (positions 16s..16s+15) and each plane, lane l = 16j + m (row
16s + m, lane group j) holds the row's bytes of that plane for lane group j (the
NB pieces (j, b), NB * w bytes); lanes are interleaved in units of
min(16, NB * w) bytes: [chunk][lane][unit]. Subtile s, plane p starts at byte
512 * (N * s + sum of the widths before p). Then the NB x 32 fp16 scales,
[block][position]. Tile bytes = 32 * NB * (4N + 2).

V tiles (body, and the q8_0 ring): 32 consecutive positions of one KV head. For
lane l in 0..63 (d16 = l % 16, j = l // 16) and n-tile n in 0..D/16-1, piece
(l, n) holds channel 16*n + d16 at tile positions T(j, i) = 4j + i (i < 4) and
16 + 4j + (i - 4) (i >= 4). For each plane, lane l's bytes are its pieces for
n = 0..NT-1 (NT * w bytes); they are interleaved across lanes in units of
u = min(16, NT * w) bytes: [chunk][lane][u]. Then the NB x 32 fp16 scales,
[block][position]. Tile bytes = 32 * NB * (4N + 2).

qN_1 bodies (codes with a scale and a minimum per block): the codes are placed as
above (u itself, 0 .. 2^N - 1, is what the planes hold); a K or V row ends with the NB
fp16 scales and then the NB fp16 minima, both in block order (row bytes
NB * (4N + 4)); a K tile ends with the scales [block][position] and then the
minima [position][block]; a V tile with the scales and then the minima, both
[block][position] (tile bytes 32 * NB * (4N + 4)).

Token-axis K (KIVI-style; Qwen3.8-27B page, reader comment on quantizing K along the token
axis): a K block is the 32 positions of one channel within a position tile. The codes of a
K tile are placed as above; the tile ends with the D fp16 scales [channel] (and, for a qN_1
K, the D fp16 minima [channel]): the same bytes as a per-token tile.

bf16 tail ring (tile layout): K tiles of 32 slots hold, for subtile s and block b,
lane l = 16j + m's 8 bf16 values of channels 32b + 8j .. +7 of slot 16s + m:
[s][b][lane][8 x bf16]; V tiles hold, for n-tile n and lane l, the 8 bf16 values
of channel 16*n + d16 at tile positions T(j, i): [n][lane][8 x bf16].

Row layout (a cache option for sparse layers): V is stored exactly like K, one
row per position (body and q8_0 ring: the K row format above; bf16 / f16 ring: the
D 16-bit values), and the rows are position-major: for each position, for each KV
head, the K row and then the V row. One position of every KV head is one contiguous
run (q8_0 with 2 KV heads: 1,088 bytes), so a gather of listed positions reads whole
runs. The body region holds [capacity32][head][K row, V row] and the ring region
[R][head][K row, V row]; the separate V regions are empty.

Arena: slabs of [layer][sequence]; each slab holds, in order and 256-byte
aligned: K body [head][capacity32/32][tile], V body [head][capacity32/32][tile],
K ring [head][R/32][tile], V ring [head][R/32][tile] (row layout: [head][.][row]
for K, and for V as well), KVarN sigma [head][K,V][D] fp16, and (when the cache
carries an indexer) the pooled index keys [capacity32][32] bf16, 64 bytes per
position (offload page: 1 x (128 / 4) x 2 bytes per token and layer).
capacity32 is the capacity rounded up to 32; R = W + S (ring slots).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
TILE = 32

_PLANES = {2: [(2, 0)], 3: [(2, 0), (1, 2)], 4: [(4, 0)], 5: [(4, 0), (1, 4)],
           6: [(4, 0), (2, 4)], 7: [(4, 0), (2, 4), (1, 6)], 8: [(8, 0)]}


def planes(n_bits: int):
    """[(width, shift)] bit planes of an N-bit code, least significant first."""
    return list(_PLANES[n_bits])


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def row_bytes(n_bits: int, head_dim: int, with_min: bool = False) -> int:
    """Bytes of one K or V row: NB * (4N + 2), plus 2 * NB for the minima of a qN_1 row."""
    nb = head_dim // BLOCK
    return nb * (4 * n_bits + 2 + (2 if with_min else 0))


def tile_positions() -> np.ndarray:
    """T[j, i]: tile position held by lane group j at element i."""
    t = np.zeros((4, 8), dtype=np.int64)
    for j in range(4):
        for i in range(8):
            t[j, i] = 4 * j + i if i < 4 else 16 + 4 * j + (i - 4)
    return t


# ----------------------------------------------------------------------------- pieces

def _piece_shifts(w: int) -> np.ndarray:
    per = 4 // w
    s = np.zeros((per, 8), dtype=np.uint64)
    for p in range(per):
        for i in range(8):
            s[p, i] = 16 * (i % 2) + 4 * w * p + w * (i // 2)
    return s


def pack_pieces(vals: np.ndarray, w: int) -> np.ndarray:
    """vals [..., M, 8] (each < 2^w) -> bytes [..., M * w]."""
    vals = np.asarray(vals)
    m = vals.shape[-2]
    if w == 8:
        return vals.astype(np.uint8).reshape(*vals.shape[:-2], m * 8)
    per = 4 // w
    assert m % per == 0
    v = vals.astype(np.uint64).reshape(*vals.shape[:-2], m // per, per, 8)
    words = np.sum(v << _piece_shifts(w), axis=(-2, -1)).astype(np.uint32)
    return np.ascontiguousarray(words).view(np.uint8).reshape(*vals.shape[:-2], m * w)


def unpack_pieces(b: np.ndarray, w: int, m: int) -> np.ndarray:
    """Inverse of pack_pieces: bytes [..., M * w] -> vals [..., M, 8]."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if w == 8:
        return b.reshape(*b.shape[:-1], m, 8)
    per = 4 // w
    words = b.reshape(*b.shape[:-1], m * w // 4, 4).copy().view(np.uint32)[..., 0].astype(np.uint64)
    v = (words[..., None, None] >> _piece_shifts(w)) & np.uint64((1 << w) - 1)
    return v.reshape(*b.shape[:-1], m, 8).astype(np.uint8)


# ----------------------------------------------------------------------------- K rows

def pack_k_rows(u: np.ndarray, d16: np.ndarray, n_bits: int, m16=None) -> np.ndarray:
    """Codes u [..., D] (uint8), scales d16 [..., D/32] and (qN_1) minima m16 [..., D/32] -> K rows
    [..., row_bytes]."""
    u = np.asarray(u, dtype=np.uint8)
    d = u.shape[-1]
    nb = d // BLOCK
    pieces = u.reshape(*u.shape[:-1], nb, 4, 8)            # [.., b, j, i]
    pieces = np.swapaxes(pieces, -3, -2)                    # [.., j, b, i]
    parts = []
    for w, sh in planes(n_bits):
        v = (pieces >> sh) & ((1 << w) - 1)
        parts.append(pack_pieces(v, w).reshape(*u.shape[:-1], 4 * nb * w))
    parts.append(np.ascontiguousarray(np.asarray(d16, dtype=np.float16)).view(np.uint8)
                 .reshape(*u.shape[:-1], 2 * nb))
    if m16 is not None:
        parts.append(np.ascontiguousarray(np.asarray(m16, dtype=np.float16)).view(np.uint8)
                     .reshape(*u.shape[:-1], 2 * nb))
    return np.concatenate(parts, axis=-1)


def unpack_k_rows(rows: np.ndarray, n_bits: int, head_dim: int):
    """K rows [..., row_bytes] -> (u [..., D], d16 [..., D/32]) (the minima of a qN_1 row follow the scales)."""
    rows = np.asarray(rows, dtype=np.uint8)
    nb = head_dim // BLOCK
    lead = rows.shape[:-1]
    u = np.zeros((*lead, 4, nb, 8), dtype=np.uint8)
    off = 0
    for w, sh in planes(n_bits):
        sz = 4 * nb * w
        v = unpack_pieces(rows[..., off:off + sz].reshape(*lead, 4, nb * w), w, nb)
        u |= (v << sh).astype(np.uint8)
        off += sz
    d16 = np.ascontiguousarray(rows[..., off:off + 2 * nb]).view(np.float16)
    u = np.swapaxes(u, -3, -2).reshape(*lead, head_dim)
    return u, d16


# ----------------------------------------------------------------------------- K tiles

def _k_tile_parts(n_bits: int, head_dim: int):
    """[(subtile, row byte offset of the plane, lane run bytes NB * w)] in tile order."""
    nb = head_dim // BLOCK
    parts = []
    for s in range(2):
        off = 0
        for w, _ in planes(n_bits):
            parts.append((s, off, nb * w))
            off += 4 * nb * w
    return parts


def pack_k_tiles(u: np.ndarray, d16: np.ndarray, n_bits: int, m16=None) -> np.ndarray:
    """Codes u [n_tiles, 32, D], scales [n_tiles, 32, D/32] and (qN_1) minima [n_tiles, 32, D/32] -> K tiles
    [n_tiles, tile_bytes]."""
    u = np.asarray(u, dtype=np.uint8)
    ntl, tt, d = u.shape
    assert tt == TILE
    nb = d // BLOCK
    rows = pack_k_rows(u, d16, n_bits)                       # [ntl, 32, row_bytes]
    out = []
    for s, off, lb in _k_tile_parts(n_bits, d):
        sub = rows[:, 16 * s:16 * s + 16, :]                 # [ntl, m, row]
        # lane l = 16 j + m takes row m's run of lane group j: bytes off + j*lb .. + lb
        runs = np.stack([sub[:, :, off + j * lb: off + (j + 1) * lb] for j in range(4)], axis=1)  # [ntl, j, m, lb]
        runs = runs.reshape(ntl, 64, lb)
        cu = min(16, lb)
        out.append(runs.reshape(ntl, 64, lb // cu, cu).transpose(0, 2, 1, 3).reshape(ntl, 64 * lb))
    sc = np.ascontiguousarray(np.asarray(d16, dtype=np.float16).transpose(0, 2, 1))   # [ntl, b, t]
    out.append(sc.view(np.uint8).reshape(ntl, 2 * nb * TILE))
    if m16 is not None:   # minima [position][block]
        out.append(np.ascontiguousarray(np.asarray(m16, dtype=np.float16)).view(np.uint8).reshape(ntl, 2 * nb * TILE))
    return np.concatenate(out, axis=-1)


def pack_k_tiles_token_axis(u: np.ndarray, d16: np.ndarray, n_bits: int, m16=None) -> np.ndarray:
    """Token-axis K: codes u [n_tiles, 32, D], scales d16 [n_tiles, D] (one per channel and tile) and (qN_1)
    minima [n_tiles, D] -> K tiles [n_tiles, tile_bytes]: the codes placed as in a per-token tile, then the
    scales [channel], then the minima [channel]."""
    u = np.asarray(u, dtype=np.uint8)
    ntl, _, d = u.shape
    codes = pack_k_tiles(u, np.zeros((ntl, TILE, d // BLOCK), dtype=np.float16), n_bits)[:, :TILE * d * n_bits // 8]
    parts = [codes, np.ascontiguousarray(np.asarray(d16, dtype=np.float16)).view(np.uint8).reshape(ntl, 2 * d)]
    if m16 is not None:
        parts.append(np.ascontiguousarray(np.asarray(m16, dtype=np.float16)).view(np.uint8).reshape(ntl, 2 * d))
    return np.concatenate(parts, axis=-1)


def unpack_k_tiles(tiles: np.ndarray, n_bits: int, head_dim: int):
    """K tiles [n_tiles, tile_bytes] -> (u [n_tiles, 32, D], d16 [n_tiles, 32, D/32])."""
    tiles = np.asarray(tiles, dtype=np.uint8)
    ntl = tiles.shape[0]
    nb = head_dim // BLOCK
    rb = row_bytes(n_bits, head_dim)
    rows = np.zeros((ntl, TILE, rb), dtype=np.uint8)
    pos = 0
    for s, off, lb in _k_tile_parts(n_bits, head_dim):
        cu = min(16, lb)
        x = tiles[:, pos:pos + 64 * lb].reshape(ntl, lb // cu, 64, cu).transpose(0, 2, 1, 3).reshape(ntl, 4, 16, lb)
        for j in range(4):
            rows[:, 16 * s:16 * s + 16, off + j * lb: off + (j + 1) * lb] = x[:, j]
        pos += 64 * lb
    d16 = np.ascontiguousarray(tiles[:, pos:pos + 2 * nb * TILE]).view(np.float16).reshape(ntl, nb, TILE)
    d16 = np.ascontiguousarray(d16.transpose(0, 2, 1))
    rows[:, :, 4 * nb * n_bits:] = np.ascontiguousarray(d16).view(np.uint8).reshape(ntl, TILE, 2 * nb)
    u, _ = unpack_k_rows(rows, n_bits, head_dim)
    return u, d16


def pack_bf16_k_tiles(bits: np.ndarray) -> np.ndarray:
    """bf16 bits [n_tiles, 32, D] -> bf16 ring K tiles [n_tiles, 64 * D] bytes ([s][b][lane][8])."""
    bits = np.asarray(bits, dtype=np.uint16)
    ntl, _, d = bits.shape
    nb = d // BLOCK
    x = bits.reshape(ntl, 2, 16, nb, 4, 8)                   # [ntl, s, m, b, j, i]
    x = x.transpose(0, 1, 3, 4, 2, 5)                        # [ntl, s, b, j, m, i] -> lane = 16 j + m
    return np.ascontiguousarray(x).view(np.uint8).reshape(ntl, -1)


def unpack_bf16_k_tiles(tiles: np.ndarray, head_dim: int) -> np.ndarray:
    tiles = np.ascontiguousarray(tiles, dtype=np.uint8)
    ntl = tiles.shape[0]
    nb = head_dim // BLOCK
    x = tiles.view(np.uint16).reshape(ntl, 2, nb, 4, 16, 8).transpose(0, 1, 4, 2, 3, 5)
    return np.ascontiguousarray(x).reshape(ntl, TILE, head_dim)


# ----------------------------------------------------------------------------- V tiles

def _v_gather_index(head_dim: int):
    nt = head_dim // 16
    tp = tile_positions()
    lane = np.arange(64)
    t_idx = tp[lane // 16][:, None, :].repeat(nt, axis=1)                  # [64, NT, 8]
    d_idx = (16 * np.arange(nt)[None, :, None] + (lane % 16)[:, None, None]).repeat(8, axis=2)
    return t_idx, d_idx


def pack_v_tiles(u: np.ndarray, d16: np.ndarray, n_bits: int, m16=None) -> np.ndarray:
    """Codes u [n_tiles, 32, D], scales [n_tiles, 32, D/32] and (qN_1) minima -> tiles [n_tiles, tile_bytes]."""
    u = np.asarray(u, dtype=np.uint8)
    ntl, tt, d = u.shape
    assert tt == TILE
    nt = d // 16
    t_idx, d_idx = _v_gather_index(d)
    g = u[:, t_idx, d_idx]                                  # [ntl, 64, NT, 8]
    parts = []
    for w, sh in planes(n_bits):
        v = (g >> sh) & ((1 << w) - 1)
        lane_bytes = pack_pieces(v, w)                      # [ntl, 64, NT*w]
        lb = nt * w
        cu = min(16, lb)
        x = lane_bytes.reshape(ntl, 64, lb // cu, cu).transpose(0, 2, 1, 3)
        parts.append(x.reshape(ntl, 64 * lb))
    sc = np.ascontiguousarray(np.asarray(d16, dtype=np.float16).transpose(0, 2, 1))   # [ntl, b, t]
    parts.append(sc.view(np.uint8).reshape(ntl, -1))
    if m16 is not None:   # minima [block][position]
        mn = np.ascontiguousarray(np.asarray(m16, dtype=np.float16).transpose(0, 2, 1))
        parts.append(mn.view(np.uint8).reshape(ntl, -1))
    return np.concatenate(parts, axis=-1)


def unpack_v_tiles(tiles: np.ndarray, n_bits: int, head_dim: int):
    """Tiles [n_tiles, tile_bytes] -> (u [n_tiles, 32, D], d16 [n_tiles, 32, D/32])."""
    tiles = np.asarray(tiles, dtype=np.uint8)
    ntl = tiles.shape[0]
    nt = head_dim // 16
    nb = head_dim // BLOCK
    g = np.zeros((ntl, 64, nt, 8), dtype=np.uint8)
    off = 0
    for w, sh in planes(n_bits):
        lb = nt * w
        cu = min(16, lb)
        x = tiles[:, off:off + 64 * lb].reshape(ntl, lb // cu, 64, cu).transpose(0, 2, 1, 3)
        v = unpack_pieces(x.reshape(ntl, 64, lb), w, nt)
        g |= (v << sh).astype(np.uint8)
        off += 64 * lb
    t_idx, d_idx = _v_gather_index(head_dim)
    u = np.zeros((ntl, TILE, head_dim), dtype=np.uint8)
    u[:, t_idx, d_idx] = g
    d16 = np.ascontiguousarray(tiles[:, off:off + TILE * nb * 2]).view(np.float16).reshape(ntl, nb, TILE)
    return u, np.ascontiguousarray(d16.transpose(0, 2, 1))


def pack_bf16_v_tiles(bits: np.ndarray) -> np.ndarray:
    """bf16 bits [n_tiles, 32, D] -> bf16 ring V tiles [n_tiles, 64 * D] bytes ([n][lane][8])."""
    bits = np.asarray(bits, dtype=np.uint16)
    ntl, _, d = bits.shape
    t_idx, d_idx = _v_gather_index(d)                       # [64, NT, 8]
    g = bits[:, t_idx, d_idx]                               # [ntl, 64, NT, 8]
    g = g.transpose(0, 2, 1, 3)                             # [ntl, NT, 64, 8]
    return np.ascontiguousarray(g).view(np.uint8).reshape(ntl, -1)


def unpack_bf16_v_tiles(tiles: np.ndarray, head_dim: int) -> np.ndarray:
    tiles = np.ascontiguousarray(tiles, dtype=np.uint8)
    ntl = tiles.shape[0]
    nt = head_dim // 16
    g = tiles.view(np.uint16).reshape(ntl, nt, 64, 8).transpose(0, 2, 1, 3)
    t_idx, d_idx = _v_gather_index(head_dim)
    out = np.zeros((ntl, TILE, head_dim), dtype=np.uint16)
    out[:, t_idx, d_idx] = g
    return out


# ----------------------------------------------------------------------------- arena

def ring_slots(cfg: dict) -> int:
    return cfg["tail_len"] + cfg["tail_slack"] if cfg["tail_len"] > 0 else 0


def slab_layout(cfg: dict) -> dict:
    """Byte offsets and sizes of the regions of one (layer, sequence) slab."""
    d = cfg["head_dim"]
    hk = cfg["n_kv_heads"]
    cap32 = _round_up(cfg["capacity"], TILE)
    rk = row_bytes(cfg["k_bits"], d, bool(cfg.get("k_min", 0)))
    rv = row_bytes(cfg["v_bits"], d, bool(cfg.get("v_min", 0)))
    r = ring_slots(cfg)
    if cfg["tail_len"] > 0 and cfg["tail_dtype"] in (1, 3):   # bf16 or f16 values
        ring_rk = ring_rv = 2 * d
    elif cfg["tail_len"] > 0 and cfg["tail_dtype"] == 2:
        ring_rk = ring_rv = row_bytes(8, d)
    else:
        ring_rk = ring_rv = 0
    rows = cfg.get("layout", 0) == 1     # position-major K and V rows in the K regions
    sizes = {
        "k_body": hk * cap32 * (rk + rv if rows else rk),
        "v_body": 0 if rows else hk * cap32 * rv,
        "k_ring": hk * r * (ring_rk + ring_rv if rows else ring_rk),
        "v_ring": 0 if rows else hk * r * ring_rv,
        "sigma": hk * 2 * d * 2 if cfg["kvarn"] else 0,
        "index": cap32 * 64 if cfg.get("index_dim", 0) else 0,
    }
    off = 0
    lay = {}
    for name in ("k_body", "v_body", "k_ring", "v_ring", "sigma", "index"):
        off = _round_up(off, 256)
        lay[name] = (off, sizes[name])
        off += sizes[name]
    lay["slab"] = _round_up(off, 256)
    lay["cap32"] = cap32
    lay["row_k"] = rk
    lay["row_v"] = rv
    lay["ring_row_k"] = ring_rk
    lay["ring_row_v"] = ring_rv
    lay["ring_slots"] = r
    return lay


def cache_bytes(cfg: dict) -> int:
    """Exact arena bytes: n_layers * max_seqs slabs."""
    return cfg["n_layers"] * cfg["max_seqs"] * slab_layout(cfg)["slab"]
