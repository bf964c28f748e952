// Arena format shared by the kvq host code and kernels.
//
// The pages fix only the size of a qN_0 block (N bits per value, one fp16 scale per 32 values; BeeLlama
// page KV MiB table, KVarN benchmark page cache-size column). The placement of the bits is ours and is
// chosen so that the decode kernel loads MFMA operands with wide, coalesced loads and no transposes:
//
// * An N-bit biased code u = c + 2^(N-1) is split into bit planes (least significant first):
//   2:[2] 3:[2,1] 4:[4] 5:[4,1] 6:[4,2] 7:[4,2,1] 8:[8].
// * A piece is 8 codes e0..e7 of one plane. For plane width w in {1,2,4}, 4/w pieces share a 32-bit
//   little-endian word and element i of piece p sits at bit 16*(i&1) + 4*w*p + w*(i>>1), so that the
//   pair (e_2k, e_2k+1) always lands in the two 16-bit halves at the same offset (one AND-OR forms two
//   fp16 "1024 + value" magic numbers). For w = 8 a piece is 8 bytes, e_i in byte i.
// * K rows, one per (position, KV head): per plane, for lane group j = 0..3 the pieces of blocks
//   b = 0..NB-1 (piece (j,b) = channels 32b+8j+i), then NB fp16 scales. The row layout stores them as is.
// * K tiles (tile layout, body and q8_0 ring): the K rows of 32 positions rearranged for 1 KiB loads: for
//   subtile s (positions 16s..16s+15) and plane p, lane l = 16j + m holds row 16s+m's run of lane group j
//   (NB*w bytes) as [chunk][lane][min(16, NB*w)] starting at byte 512*(N*s + widths before p); then the
//   NB x 32 fp16 scales [block][position].
// * V tiles (body and q8_0 ring), 32 positions of one KV head: per plane, lane l (d16 = l&15,
//   j = l>>4) owns pieces n = 0..NT-1, piece (l,n) = channel 16n+d16 at tile positions
//   T(j,i) = 4j+i (i<4), 16+4j+i-4 (i>=4); lanes' bytes are interleaved in units of
//   min(16, NT*w) bytes ([chunk][lane][unit]); then the NB x 32 fp16 scales [block][position].
// * qN_1 bodies (a scale and a minimum per block; the planes hold the code u in 0..2^N-1 itself): a row ends
//   with the NB scales and then the NB fp16 minima; a K tile with the scales [block][position] and then the
//   minima [position][block] (the MFMA A operand of the minimum term: one 16-byte run per position); a V tile
//   with the scales and the minima, both [block][position].
// * bf16 tail ring: K tiles hold, per subtile s and block b, lane (j, m)'s 8 bf16 values of channels
//   32b+8j.. of slot 16s+m: [s][b][lane][8 x bf16]; V tiles hold, per n-tile and lane, the 8 bf16 values
//   of channel 16n+d16 at positions T(j,i): [n][lane][8 x bf16].
// * Row layout (a cache option for sparse layers): V is stored exactly like K, one row per position
//   (body, q8_0 ring) or plain 16-bit rows (bf16 / f16 ring), position-major: for each position, for each KV
//   head, the K row and then the V row, so one position of every head is one contiguous run. The body region
//   holds [cap32][head][K row, V row], the ring region [R][head][K row, V row]; the V regions are empty.
// * Arena: [layer][seq] slabs; a slab holds (256-byte aligned) K body [head][cap32/32][tile],
//   V body [head][cap32/32][tile], K ring [head][R/32][tile], V ring [head][R/32][tile] (row layout:
//   [head][positions][row] for K and V), KVarN sigma [head][K,V][D] fp16, and for a cache with an indexer the
//   pooled index keys [cap32][32] bf16 (64 bytes per position: offload page, 1 x (128 / 4) x 2 bytes).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef KVQ_HD
#if defined(__HIPCC__)
#define KVQ_HD __host__ __device__ inline
#else
#define KVQ_HD inline
#endif
#endif

namespace kvq {

constexpr int kTile = 32;        // positions per V tile
constexpr int kBlock = 32;       // values per quantization block
constexpr int kIndexWidth = 32;  // pooled index key values per position (indexer head dim / pooling ratio)

// Planes of an N-bit code: count, widths and shifts (least significant plane first).
KVQ_HD int plane_count(int n) { return (n == 7) ? 3 : (n == 3 || n == 5 || n == 6) ? 2 : 1; }
KVQ_HD int plane_width(int n, int p) {
  switch (n) {
    case 2: return 2;
    case 3: return p == 0 ? 2 : 1;
    case 4: return 4;
    case 5: return p == 0 ? 4 : 1;
    case 6: return p == 0 ? 4 : 2;
    case 7: return p == 0 ? 4 : (p == 1 ? 2 : 1);
    default: return 8;
  }
}
KVQ_HD int plane_shift(int n, int p) {
  switch (n) {
    case 3: return p == 0 ? 0 : 2;
    case 5: return p == 0 ? 0 : 4;
    case 6: return p == 0 ? 0 : 4;
    case 7: return p == 0 ? 0 : (p == 1 ? 4 : 6);
    default: return 0;
  }
}
// Bytes of all planes before plane p, for `pieces` pieces per plane.
KVQ_HD int plane_offset(int n, int p, int pieces) {
  int off = 0;
  for (int q = 0; q < p; ++q) off += plane_width(n, q) * pieces;
  return off;
}

KVQ_HD size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }
// with_min: a qN_1 row (one fp16 minimum per block after the scales)
KVQ_HD int row_bytes(int n_bits, int head_dim, int with_min = 0) {
  return head_dim / kBlock * (4 * n_bits + 2 + (with_min ? 2 : 0));
}
KVQ_HD int tile_bytes(int n_bits, int head_dim, int with_min = 0) { return kTile * row_bytes(n_bits, head_dim, with_min); }
KVQ_HD int tile_pos(int j, int i) { return i < 4 ? 4 * j + i : 16 + 4 * j + (i - 4); }

// Offset of lane l's byte `b` of its run of `lb` bytes in a lane-interleaved tile part: runs are stored in
// units of min(16, lb) bytes, [unit index][lane][unit].
KVQ_HD int lane_run_byte(int lane, int b, int lb) {
  int unit = lb < 16 ? lb : 16;
  return (b / unit) * 64 * unit + lane * unit + (b % unit);
}

// Offset of lane l's byte `b` (within its per-plane run of nt*w bytes) in a V tile's plane.
KVQ_HD int vtile_lane_byte(int lane, int b, int nt, int w) {
  int lb = nt * w;
  int unit = lb < 16 ? lb : 16;
  return (b / unit) * 64 * unit + lane * unit + (b % unit);
}

// Row layout: byte offsets (within the body or ring region) of the K row of (position or slot p, head h) and
// of its V row; pair = row_k + row_v (or ring_row_k + ring_row_v).
KVQ_HD size_t rows_k_off(size_t p, int h, int n_kv_heads, int pair) { return (p * n_kv_heads + h) * (size_t)pair; }
KVQ_HD size_t rows_v_off(size_t p, int h, int n_kv_heads, int pair, int row_k) {
  return rows_k_off(p, h, n_kv_heads, pair) + row_k;
}

struct SlabLayout {
  size_t k_body, v_body, k_ring, v_ring, sigma, index;   // region offsets within a slab
  size_t k_body_sz, v_body_sz, k_ring_sz, v_ring_sz, sigma_sz, index_sz;
  size_t slab;                                           // slab bytes (256-aligned)
  int cap32, row_k, row_v, ring_row_k, ring_row_v, ring_slots;
};

// tail_dtype: 0 none, 1 bf16, 2 q8_0, 3 f16. index: 0 none, else the cache holds pooled index keys.
// k_min / v_min: qN_1 bodies.
KVQ_HD SlabLayout slab_layout(int capacity, int n_kv_heads, int head_dim, int k_bits, int v_bits,
                              int kvarn, int tail_len, int tail_slack, int tail_dtype, int index, int k_min = 0,
                              int v_min = 0, int rows = 0) {
  SlabLayout L{};
  L.cap32 = (int)round_up((size_t)capacity, kTile);
  L.row_k = row_bytes(k_bits, head_dim, k_min);
  L.row_v = row_bytes(v_bits, head_dim, v_min);
  L.ring_slots = tail_len > 0 ? tail_len + tail_slack : 0;
  if (tail_len > 0 && (tail_dtype == 1 || tail_dtype == 3)) {   // 16-bit values
    L.ring_row_k = L.ring_row_v = 2 * head_dim;
  } else if (tail_len > 0 && tail_dtype == 2) {
    L.ring_row_k = L.ring_row_v = row_bytes(8, head_dim);
  }
  size_t hk = (size_t)n_kv_heads;
  if (rows) {   // position-major K and V rows in the K regions
    L.k_body_sz = hk * L.cap32 * (L.row_k + L.row_v);
    L.v_body_sz = 0;
    L.k_ring_sz = hk * L.ring_slots * (L.ring_row_k + L.ring_row_v);
    L.v_ring_sz = 0;
  } else {
    L.k_body_sz = hk * L.cap32 * L.row_k;
    L.v_body_sz = hk * L.cap32 * L.row_v;
    L.k_ring_sz = hk * L.ring_slots * L.ring_row_k;
    L.v_ring_sz = hk * L.ring_slots * L.ring_row_v;
  }
  L.sigma_sz = kvarn ? hk * 2 * head_dim * 2 : 0;
  L.index_sz = index ? (size_t)L.cap32 * kIndexWidth * 2 : 0;
  size_t off = 0;
  L.k_body = off; off = round_up(off + L.k_body_sz, 256);
  L.v_body = off; off = round_up(off + L.v_body_sz, 256);
  L.k_ring = off; off = round_up(off + L.k_ring_sz, 256);
  L.v_ring = off; off = round_up(off + L.v_ring_sz, 256);
  L.sigma = off; off = round_up(off + L.sigma_sz, 256);
  L.index = off; off = round_up(off + L.index_sz, 256);
  L.slab = off;
  return L;
}

}  // namespace kvq
