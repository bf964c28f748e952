// Multi-query attention with two queries per wave, for caches without qN_1 bodies or token-axis K. The bf16 query
// times 2^-e is exact in one fp16 (an 8-bit significand inside an 11-bit one), so a wave places two queries' 8
// heads side by side in the 16 columns of the QK product (columns 0-7: its first query's heads, 8-15: its
// second's) and every K or V operand it reads from LDS serves both queries. A KVarN cache keeps this form: the
// decode multiplies its body K codes by sigma_K (KVarN benchmark page: the per-channel factor the keys are divided
// by) instead of the query, and its body V values are multiplied by sigma_V at the end. A work-group of 8 waves
// takes a block of up to 16 (KVarN: 8) consecutive query positions of one sequence and one KV head over a range
// of the block's prefix tiles.
//
// Per 32-position tile the work-group decodes the raw tile once into the operand layout of the one-query kernel
// (kvq_mq_impl.h): K codes as exact fp16 integers with the tile's fp16 K scales (KVarN body: code x sigma_K as an
// fp16 value and remainder), each V code times its block scale as an fp16 pair (rounded product, exact
// remainder). A wave then computes QK on MFMA, applies the K scale of each (position, block) in fp32, masks
// causally per column, updates its online softmax per column and runs P.V on MFMA with A = P as rows (query,
// head) split into fp16 rounded values and remainders: three products per n-tile (value x value, remainder x
// value, value x remainder; the remainder x remainder term is below the fp32 accumulation's rounding).
//
// One work-group barrier per tile: between two barriers the work-group decodes tile i + 1 into one operand buffer
// while it computes tile i from the other. Blocks of at most 8 queries compute on waves 0-3 while waves 4-7
// load (from global memory into registers, two tiles ahead) and decode; larger blocks (prefill without KVarN)
// compute and decode on every wave, the raw tile staged through LDS. 16-bit ring tiles (bf16 / f16 tails; a split
// reaches them after all its quantized tiles) need no decode: they go from registers into an operand buffer, one
// tile ahead.
#pragma once

#include "kvq_mq_impl.h"
#include "kvq_mq_plan.h"

namespace kvq {
namespace {


// The lane's share of its column's query: channels 32b + 8g .. 32b + 8g + 7 of every block b (g = lane / 16), the
// bf16 words as they are (zero for an unused column). The four lanes of a column together hold its whole row, so
// the wave's 64 lanes hold both queries' heads: one batch of loads serves the exponent shift and the operand.
__device__ inline void pair_query_words(const uint16_t* qrow, bool col_ok, u32x4* qw) {
  const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int b = 0; b < 8; ++b) qw[b] = col_ok ? *(const u32x4*)(qrow + 32 * b + 8 * gq) : u32x4{0u, 0u, 0u, 0u};
}

// Exponent shift of the wave's queries: their largest |q| brought below 2^9.
__device__ inline int pair_query_shift(const u32x4* qw) {
  float amax = 0.0f;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(qw[b][k] << 16)), fabsf(__uint_as_float(qw[b][k] & 0xFFFF0000u))));
  amax = wave_max_16_32(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  return amax > 0.0f ? ilogbf(amax) - 8 : 0;
}

// Query operand of block b: the words times 2^-e in fp16, or (`bf16`, for a bf16 ring) the bf16 words as they are.
__device__ inline half8 pair_qop(const u32x4& qw, int e, bool bf16) {
  if (bf16) return __builtin_bit_cast(half8, qw);
  half8 out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = (_Float16)ldexpf(__uint_as_float(qw[k] << 16), -e);
    out[2 * k + 1] = (_Float16)ldexpf(__uint_as_float(qw[k] & 0xFFFF0000u), -e);
  }
  return out;
}

// QK of a quantized tile (qN_0 body or q8_0 ring): one MFMA per (block, 16-row subtile) (KLO: two, the K operand
// as fp16 value and remainder: KVarN body codes times sigma_K), the K scale of each (position, block) applied to
// the fp32 result. x[4s + r]: position 16s + 4g + r of the lane's column.
// The LDS reads of a group of blocks are issued together, ahead of their MFMAs, so their latencies overlap.
template <bool KLO, class Ops>
__device__ inline void pair_qk_q(const Ops& ops, const half8* qop, float qmul, float* x) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float sc[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  constexpr int G = 8;   // blocks per group
#pragma unroll
  for (int b0 = 0; b0 < 8; b0 += G) {
    u32x4 k0[G], k1[G], l0[KLO ? G : 1], l1[KLO ? G : 1];
    u32x2 d0[G], d1[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      k0[j] = ops.k[(b0 + j) * 64 + lane];
      k1[j] = ops.k[(8 + b0 + j) * 64 + lane];
      if constexpr (KLO) {
        l0[j] = ops.kl[(b0 + j) * 64 + lane];
        l1[j] = ops.kl[(8 + b0 + j) * 64 + lane];
      }
      d0[j] = *(const u32x2*)(ops.ks + (b0 + j) * 32 + 4 * g);
      d1[j] = *(const u32x2*)(ops.ks + (b0 + j) * 32 + 16 + 4 * g);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      floatx4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, k0[j]), qop[b0 + j],
                                                          floatx4{0, 0, 0, 0}, 0, 0, 0);
      floatx4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, k1[j]), qop[b0 + j],
                                                          floatx4{0, 0, 0, 0}, 0, 0, 0);
      if constexpr (KLO) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, l0[j]), qop[b0 + j], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, l1[j]), qop[b0 + j], c1, 0, 0, 0);
      }
      sc[0][0] = fmaf(c0[0], lo_h(d0[j][0]), sc[0][0]);
      sc[0][1] = fmaf(c0[1], hi_h(d0[j][0]), sc[0][1]);
      sc[0][2] = fmaf(c0[2], lo_h(d0[j][1]), sc[0][2]);
      sc[0][3] = fmaf(c0[3], hi_h(d0[j][1]), sc[0][3]);
      sc[1][0] = fmaf(c1[0], lo_h(d1[j][0]), sc[1][0]);
      sc[1][1] = fmaf(c1[1], hi_h(d1[j][0]), sc[1][1]);
      sc[1][2] = fmaf(c1[2], lo_h(d1[j][1]), sc[1][2]);
      sc[1][3] = fmaf(c1[3], hi_h(d1[j][1]), sc[1][3]);
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * s + r] = sc[s][r] * qmul;
}

// QK of a 16-bit ring tile (bf16 values with bf16 MFMA, f16 values with fp16 MFMA).
template <bool F16, class Ops>
__device__ inline void pair_qk_16(const Ops& ops, const half8* qop, float qmul, float* x) {
  const int lane = threadIdx.x & 63;
  floatx4 c[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  constexpr int G = 4;
#pragma unroll
  for (int b0 = 0; b0 < 8; b0 += G) {
    u32x4 kk[2][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      kk[0][j] = ops.k[(b0 + j) * 64 + lane];
      kk[1][j] = ops.k[(8 + b0 + j) * 64 + lane];
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if constexpr (F16)
          c[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, kk[s][j]), qop[b0 + j], c[s], 0, 0, 0);
        else
          c[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[s][j]),
                                                         __builtin_bit_cast(bf16x8, qop[b0 + j]), c[s], 0, 0, 0);
      }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * s + r] = c[s][r] * qmul;
}

// P.V of a quantized tile: A = P (rows: the wave's (query, head) columns) as fp16 rounded values and remainders,
// against the scaled V values and their remainders.
template <class Ops>
__device__ inline void pair_pv_q(WaveState& st, const Ops& ops, const float* p) {
  const int lane = threadIdx.x & 63;
  half8 ah, al;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)p[i];
    ah[i] = h;
    al[i] = (_Float16)(p[i] - (float)h);
  }
  // n-tiles in groups of 4, the next group's LDS reads issued before this group's MFMAs (each accumulator's three
  // products 4 apart)
  constexpr int G = 4;
  half8 v[2][G], vl[2][G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    v[0][j] = __builtin_bit_cast(half8, ops.v[j * 64 + lane]);
    vl[0][j] = __builtin_bit_cast(half8, ops.vl[j * 64 + lane]);
  }
#pragma unroll
  for (int n0 = 0; n0 < 16; n0 += G) {
    const int cb = (n0 / G) & 1;
    if (n0 + G < 16) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        v[cb ^ 1][j] = __builtin_bit_cast(half8, ops.v[(n0 + G + j) * 64 + lane]);
        vl[cb ^ 1][j] = __builtin_bit_cast(half8, ops.vl[(n0 + G + j) * 64 + lane]);
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
      st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, v[cb][j], st.o[n0 + j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < G; ++j)
      st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, v[cb][j], st.o[n0 + j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < G; ++j)
      st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, vl[cb][j], st.o[n0 + j], 0, 0, 0);
  }
}

// P.V of a 16-bit ring tile: P as rounded values and remainders in the ring's type, against the stored values.
template <bool F16, class Ops>
__device__ inline void pair_pv_16(WaveState& st, const Ops& ops, const float* p) {
  const int lane = threadIdx.x & 63;
  if constexpr (F16) {
    half8 ah, al;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const _Float16 h = (_Float16)p[i];
      ah[i] = h;
      al[i] = (_Float16)(p[i] - (float)h);
    }
#pragma unroll
    for (int n0 = 0; n0 < 16; n0 += 4) {
      half8 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __builtin_bit_cast(half8, ops.v[(n0 + j) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < 4; ++j) st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, v[j], st.o[n0 + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, v[j], st.o[n0 + j], 0, 0, 0);
    }
  } else {
    bf16x8 ah, al;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)p[i];
      ah[i] = h;
      al[i] = (__bf16)(p[i] - (float)h);
    }
#pragma unroll
    for (int n0 = 0; n0 < 16; n0 += 4) {
      bf16x8 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = __builtin_bit_cast(bf16x8, ops.v[(n0 + j) * 64 + lane]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, v[j], st.o[n0 + j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st.o[n0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, v[j], st.o[n0 + j], 0, 0, 0);
    }
  }
}

// Where the tiles of one (sequence, KV head) live: tile_ref's addressing with the per-head bases precomputed, held by
// value (so the decode waves' loops take no reference to the kernel's argument block).
struct TileAddr {
  const uint8_t* kbody;   // the head's body tile 0
  const uint8_t* vbody;
  const uint8_t* kring;   // the head's ring tile 0
  const uint8_t* vring;
  int tile_k, tile_v, ring_tile_k, ring_tile_v;
  int n_body, ring_t0, ring_tiles, ring_kind;

  __device__ inline TileRef operator()(int i) const {
    TileRef r;
    if (i < n_body) {
      r.k = kbody + (size_t)i * tile_k;
      r.v = vbody + (size_t)i * tile_v;
      r.kbytes = tile_k;
      r.vbytes = tile_v;
      r.kind = kKindQ;
      r.pos0 = i * kTile;
    } else {
      const int t = ring_t0 + (i - n_body);
      const int slot = t % ring_tiles;
      r.k = kring + (size_t)slot * ring_tile_k;
      r.v = vring + (size_t)slot * ring_tile_v;
      r.kbytes = ring_tile_k;
      r.vbytes = ring_tile_v;
      r.kind = ring_kind;
      r.pos0 = t * kTile;
    }
    return r;
  }
};

__device__ inline TileAddr tile_addr(const MqArgs& a, const MqSeq& S, int head, int n_body) {
  const Geometry& g = a.g;
  const uint8_t* slab = g.arena + S.slab;
  TileAddr t;
  const size_t bt = (size_t)head * (g.cap32 / kTile);
  t.kbody = slab + g.k_body + bt * g.tile_k;
  t.vbody = slab + g.v_body + bt * g.tile_v;
  t.ring_tiles = g.ring_slots / kTile;
  const size_t rt = (size_t)head * t.ring_tiles;
  t.kring = slab + g.k_ring + rt * g.ring_tile_k;
  t.vring = slab + g.v_ring + rt * g.ring_tile_v;
  t.tile_k = g.tile_k;
  t.tile_v = g.tile_v;
  t.ring_tile_k = g.ring_tile_k;
  t.ring_tile_v = g.ring_tile_v;
  t.n_body = n_body;
  t.ring_t0 = S.body_len / kTile;
  t.ring_kind = g.tail_dtype == 2 ? kKindQ8Ring : g.tail_dtype == 1 ? kKindBf16Ring : kKindF16Ring;
  return t;
}

// ---- the decode of one tile by waves 4-7 alone: wave 4 + C decodes K blocks 2C and 2C + 1 of both 16-position
// subtiles and V blocks C and C + 4, each thread loading from global memory only the words of its lane's plane
// runs that its pieces sit in (a piece: 8 codes of one plane, w bytes; the runs are [chunk][lane][unit] with 8 K
// pieces per run and unit = min(16, 8w) bytes, or 16 V pieces per run and unit = 16 bytes), three tiles ahead.

template <int W, bool KRUN>
__device__ inline uint32_t run_word(const uint8_t* plane, int lane, int wd) {
  constexpr int unit = KRUN ? (8 * W < 16 ? 8 * W : 16) : 16;
  return *(const uint32_t*)(plane + ((4 * wd) / unit * 64 + lane) * unit + (4 * wd) % unit);
}

// The words piece I of the lane's runs needs, into the run arrays at the positions decode_run_piece reads.
template <int N, int I, bool KRUN>
__device__ inline void fetch_piece_words(const uint8_t* base, int lane, uint32_t* r0, uint32_t* r1, uint32_t* r2) {
  constexpr int w0 = Planes<N>::w[0], w1 = Planes<N>::w[1], w2 = Planes<N>::w[2];
  constexpr int stride = KRUN ? 512 : 1024;   // bytes of a plane per unit of width
  if constexpr (N == 8) {
    r0[2 * I] = run_word<8, KRUN>(base, lane, 2 * I);
    r0[2 * I + 1] = run_word<8, KRUN>(base, lane, 2 * I + 1);
  } else {
    r0[I / (4 / w0)] = run_word<w0, KRUN>(base, lane, I / (4 / w0));
    if constexpr (w1 > 0) r1[I / (4 / w1)] = run_word<w1, KRUN>(base + stride * w0, lane, I / (4 / w1));
    if constexpr (w2 > 0) r2[I / (4 / w2)] = run_word<w2, KRUN>(base + stride * (w0 + w1), lane, I / (4 / w2));
  }
}

// One decode thread's share of a tile in registers: its K and V words, its V scales and (wave 4, lanes 0-31) a
// 16-byte piece of the K scales.
template <int NKt, int NVt, int C>
struct QuarterWords {
  static constexpr int a0 = Planes<NKt>::w[0], a1 = Planes<NKt>::w[1], a2 = Planes<NKt>::w[2];
  static constexpr int b0 = Planes<NVt>::w[0], b1 = Planes<NVt>::w[1], b2 = Planes<NVt>::w[2];
  uint32_t k0[2][NKt == 8 ? 16 : 2 * a0], k1[2][a1 ? 2 * a1 : 1], k2[2][a2 ? 2 * a2 : 1];
  uint32_t v0[NVt == 8 ? 32 : 4 * b0], v1[b1 ? 4 * b1 : 1], v2[b2 ? 4 * b2 : 1];
  uint32_t dv[2][4];
  u32x4 ks;

  __device__ __attribute__((always_inline)) inline void load(const TileRef& r, int lane, bool ks_lane) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      fetch_piece_words<NKt, 2 * C, true>(r.k + 512 * NKt * s, lane, k0[s], k1[s], k2[s]);
      fetch_piece_words<NKt, 2 * C + 1, true>(r.k + 512 * NKt * s, lane, k0[s], k1[s], k2[s]);
    }
    fetch_piece_words<NVt, 2 * C, false>(r.v, lane, v0, v1, v2);
    fetch_piece_words<NVt, 2 * C + 1, false>(r.v, lane, v0, v1, v2);
    fetch_piece_words<NVt, 2 * C + 8, false>(r.v, lane, v0, v1, v2);
    fetch_piece_words<NVt, 2 * C + 9, false>(r.v, lane, v0, v1, v2);
    const uint8_t* vscale = r.v + 1024 * NVt;
    const int g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // the scales of operand rows 8g..8g+7 of block C + 4h
      const int blk = C + 4 * h;
      const u32x2 d0 = *(const u32x2*)(vscale + 2 * (blk * 32 + 4 * g));
      const u32x2 d1 = *(const u32x2*)(vscale + 2 * (blk * 32 + 16 + 4 * g));
      dv[h][0] = d0[0]; dv[h][1] = d0[1]; dv[h][2] = d1[0]; dv[h][3] = d1[1];
    }
    if (ks_lane) ks = *(const u32x4*)(r.k + 1024 * NKt + 16 * lane);
  }

  // KSIG (KVarN body tiles): each K code times sigma_K of its channel as an fp16 value and remainder (exact: an
  // 8-bit code times an fp16 sigma has at most 19 significant bits); sk: sigma_K of the lane's 8 channels of
  // blocks 2C and 2C + 1
  template <bool KSIG, class Ops>
  __device__ __attribute__((always_inline)) inline void decode(Ops& ops, uint32_t magic, int lane, bool ks_lane,
                                                               const u32x4* sk) const {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int o = (s * 8 + 2 * C) * 64 + lane;
      if constexpr (KSIG) {
        const uint32_t s0[4] = {sk[0][0], sk[0][1], sk[0][2], sk[0][3]};
        const uint32_t s1[4] = {sk[1][0], sk[1][1], sk[1][2], sk[1][3]};
        scale_v_piece(decode_run_piece<NKt, 2 * C>(k0[s], k1[s], k2[s], magic), s0, ops.k[o], ops.kl[o]);
        scale_v_piece(decode_run_piece<NKt, 2 * C + 1>(k0[s], k1[s], k2[s], magic), s1, ops.k[o + 64],
                      ops.kl[o + 64]);
      } else {
        k_two_pieces<NKt, 2 * C>(k0[s], k1[s], k2[s], magic, ops.k + o);
      }
    }
    const int o0 = 2 * C * 64 + lane, o1 = 2 * (C + 4) * 64 + lane;
    scale_v_piece(decode_run_piece<NVt, 2 * C>(v0, v1, v2, magic), dv[0], ops.v[o0], ops.vl[o0]);
    scale_v_piece(decode_run_piece<NVt, 2 * C + 1>(v0, v1, v2, magic), dv[0], ops.v[o0 + 64], ops.vl[o0 + 64]);
    scale_v_piece(decode_run_piece<NVt, 2 * C + 8>(v0, v1, v2, magic), dv[1], ops.v[o1], ops.vl[o1]);
    scale_v_piece(decode_run_piece<NVt, 2 * C + 9>(v0, v1, v2, magic), dv[1], ops.v[o1 + 64], ops.vl[o1 + 64]);
    if (ks_lane) ((u32x4*)ops.ks)[lane] = ks;
  }
};

// The decode waves' side of a run of quantized tiles [t0, t1) of one kind (qN_0 body: NK / NV bits; q8_0 ring: 8 / 8):
// one barrier to publish tile t0, then per tile one barrier, matching the compute waves' loop. Tile j is decoded
// into operand buffer j % 2 in the phase before the one that computes it, from words whose loads went out at the
// end of the phase two before that (three register sets in rotation).
template <int NKt, int NVt, int C, bool KSIG, class Ops>
__device__ __attribute__((always_inline)) inline void decode_run(int t0, int t1, const TileAddr ref, Ops* s_ops,
                                                                 uint32_t magic, int lane, const u32x4* sk) {
  const bool ks_lane = C == 0 && lane < 32;
  QuarterWords<NKt, NVt, C> x, y, z;   // tiles t0 + 3m, t0 + 3m + 1, t0 + 3m + 2
  x.load(ref(t0), lane, ks_lane);
  if (t0 + 1 < t1) y.load(ref(t0 + 1), lane, ks_lane);
  if (t0 + 2 < t1) z.load(ref(t0 + 2), lane, ks_lane);
  x.template decode<KSIG>(s_ops[t0 & 1], magic, lane, ks_lane, sk);
  __syncthreads();
  // the phase that computes tile p: decode tile p + 1, then load tile p + 3 into the set tile p used (decoding
  // first, a wait for the words of tile p + 1 never covers loads issued in the same phase)
  for (int p = t0; p < t1; p += 3) {
    if (p + 1 < t1) y.template decode<KSIG>(s_ops[(p + 1) & 1], magic, lane, ks_lane, sk);
    if (p + 3 < t1) x.load(ref(p + 3), lane, ks_lane);
    __syncthreads();
    if (p + 1 >= t1) break;
    if (p + 2 < t1) z.template decode<KSIG>(s_ops[p & 1], magic, lane, ks_lane, sk);
    if (p + 4 < t1) y.load(ref(p + 4), lane, ks_lane);
    __syncthreads();
    if (p + 2 >= t1) break;
    if (p + 3 < t1) x.template decode<KSIG>(s_ops[(p + 1) & 1], magic, lane, ks_lane, sk);
    if (p + 5 < t1) z.load(ref(p + 5), lane, ks_lane);
    __syncthreads();
  }
}

template <int NKt, int NVt, bool KSIG, class Ops>
__device__ __attribute__((always_inline)) inline void decode_run_of(int c, int t0, int t1, const TileAddr ref,
                                                                    Ops* s_ops, uint32_t magic, int lane,
                                                                    const u32x4* sk) {
  switch (c) {
    case 0: decode_run<NKt, NVt, 0, KSIG>(t0, t1, ref, s_ops, magic, lane, sk); break;
    case 1: decode_run<NKt, NVt, 1, KSIG>(t0, t1, ref, s_ops, magic, lane, sk); break;
    case 2: decode_run<NKt, NVt, 2, KSIG>(t0, t1, ref, s_ops, magic, lane, sk); break;
    default: decode_run<NKt, NVt, 3, KSIG>(t0, t1, ref, s_ops, magic, lane, sk); break;
  }
}

// The 16-byte pieces t0 + nthr k (k < P) of a tile, [K tile][V tile], into registers ...
template <int P>
__device__ inline void load_part(const TileRef& r, u32x4* reg, int t0, int nthr) {
  const int nk = r.kbytes / 16, nv = r.vbytes / 16;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int c = t0 + nthr * k;
    if (c < nk) reg[k] = __builtin_nontemporal_load((const u32x4*)r.k + c);
    else if (c < nk + nv) reg[k] = __builtin_nontemporal_load((const u32x4*)r.v + (c - nk));
  }
}
// ... from registers into a raw buffer ...
template <int P>
__device__ inline void stage_part(const TileRef& r, u32x4* dst, const u32x4* reg, int t0, int nthr) {
  const int n = (r.kbytes + r.vbytes) / 16;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int c = t0 + nthr * k;
    if (c < n) dst[c] = reg[k];
  }
}
// ... or, for a 16-bit ring tile (stored in operand order), into an operand buffer.
template <int P, class Ops>
__device__ inline void store16_part(const TileRef& r, Ops& ops, const u32x4* reg, int t0, int nthr) {
  const int nk = r.kbytes / 16, nv = r.vbytes / 16;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const int c = t0 + nthr * k;
    if (c < nk) ops.k[c] = reg[k];
    else if (c < nk + nv) ops.v[c - nk] = reg[k];
  }
}

// KV: a KVarN cache. Its body K codes are decoded times sigma_K (an fp16 value and remainder per code, so the
// query needs no sigma and stays one fp16 column per head), its body V values carry 1 / sigma_V until the output is
// multiplied by sigma_V, and its blocks hold 8 queries: waves 0-3 always compute and waves 4-7 decode (the K
// remainders take the LDS the raw buffers would need).
template <int NK, int NV, bool KV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mq_pair_kernel(MqArgs a) {
  constexpr int D = 256;
  constexpr int kQ = KV ? kMqBlockSingle : kMqBlockPair;   // queries per block
  using Ops = MqOpsT<KV>;
  __shared__ Ops s_ops[2];
  __shared__ u32x4 s_raw[KV ? 1 : 2][KV ? 1 : kRawChunks];
  const Geometry& g = a.g;
  // work-group -> (sequence, query block, KV head, split)
  int si = 0;
  while (si + 1 < a.n_seqs && a.seqs[si + 1].wg_begin <= (int)blockIdx.x) ++si;
  const MqSeq& S = a.seqs[si];
  int rem = blockIdx.x - S.wg_begin;
  const int split = rem % S.n_splits;
  rem /= S.n_splits;
  const int head = rem % g.n_kv_heads;
  const int qblk = rem / g.n_kv_heads;
  const int qb0 = S.q0 + kQ * qblk;                      // first query position of the block
  const int nqb = min(kQ, S.nq - kQ * qblk);
  const int end = qb0 + nqb;                             // the block attends to positions [0, end)
  const int blen = min(S.body_len, end);
  const int n_body = (blen + kTile - 1) / kTile;
  const int n_ring = end > S.body_len ? (end + kTile - 1) / kTile - S.body_len / kTile : 0;
  const int n_tiles = n_body + n_ring;
  int tb, te;   // this split's tiles [tb, te) (n_ring_splits > 0: body and ring tiles split separately)
  {
    const int nr = S.n_ring_splits, nb = S.n_splits - nr;
    if (nr == 0) {
      tb = (int)((long)split * n_tiles / S.n_splits);
      te = (int)((long)(split + 1) * n_tiles / S.n_splits);
    } else if (split < nb) {
      tb = (int)((long)split * n_body / nb);
      te = (int)((long)(split + 1) * n_body / nb);
    } else {
      tb = n_body + (int)((long)(split - nb) * n_ring / nr);
      te = n_body + (int)((long)(split - nb + 1) * n_ring / nr);
    }
  }
  // 16-bit ring tiles come after every quantized tile of the split: [tb, tq) quantized, [tq, te) 16-bit
  const bool ring16 = g.tail_dtype == 1 || g.tail_dtype == 3;
  const int tq = ring16 ? max(tb, min(te, n_body)) : te;
  const TileAddr ref = tile_addr(a, S, head, n_body);
  // KVarN: sigma_K [D] then sigma_V [D] of this head
  const uint16_t* sig = KV ? (const uint16_t*)(g.arena + S.slab + g.sigma) + (size_t)head * 2 * D : nullptr;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int hh = m16 & 7;
  const int nqw = min(2, nqb - 2 * wave);                 // queries of this wave (<= 0: it only decodes)
  const bool active = nqw > 0;
  const int qfirst = qb0 + 2 * wave, qlast = qfirst + nqw - 1;
  // the lane's column: query 2 wave + (m16 >= 8) of the block, head m16 & 7
  const int qi = 2 * wave + (m16 >= 8 ? 1 : 0);
  const bool col_ok = active && qi < nqb && hh < a.group;
  const int qpos_col = qb0 + qi;
  const int row_base = S.row0 + kQ * qblk;
  const int qi_c = active ? min(qi, nqb - 1) : 0;         // a row inside the call's query array
  const uint16_t* qrow = a.q + ((size_t)(row_base + qi_c) * a.n_q_heads + (size_t)head * a.group +
                                (hh < a.group ? hh : 0)) * D;

  // Blocks of at most 8 queries compute on waves 0-3 only: waves 4-7 then load, stage and decode every tile
  // alone (each thread as two decode threads), in a loop of their own, so that neither role's loop holds the
  // other's registers and the decode of tile i + 1 runs on other waves of each SIMD than the compute of tile i.
  // Larger blocks (prefill) compute and decode on every wave.
  const bool apart = KV || nqb <= 8;
  // the split's first tile is on its way while the query operand is built
  u32x4 reg[3];
  if (!apart && tb < tq) load_part<3>(ref(tb), reg, tid, 512);

  half8 qop[8];
  float qmul = 0.0f;
  if (active && tb < te) {
    u32x4 qw[8];
    pair_query_words(qrow, col_ok, qw);
    const int qexp = pair_query_shift(qw);   // |q| 2^-e < 2^9
    const bool bf16 = tq == tb && g.tail_dtype == 1;   // a split of bf16 ring tiles only
#pragma unroll
    for (int b = 0; b < 8; ++b) qop[b] = pair_qop(qw[b], bf16 ? 0 : qexp, bf16);
    qmul = a.scale * kLog2e * (bf16 ? 1.0f : ldexpf(1.0f, qexp));
  }

  WaveState st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int n = 0; n < 16; ++n) st.o[n] = floatx4{0, 0, 0, 0};
  uint32_t magic = kMagic;
  asm volatile("" : "+v"(magic));

  // tile i of this wave's queries: QK, causal mask per column, online softmax, P.V
  auto compute = [&](int i, const Ops& ops) {
    if (!active) return;
    const TileRef r = ref(i);
    const bool body = r.kind == kKindQ;
    const int lo = body ? 0 : S.body_len;
    const int lim = body ? blen : end;
    if (r.pos0 >= min(lim, qlast + 1) || r.pos0 + kTile <= lo) return;
    float x[8], p[8];
    if (body) pair_qk_q<KV>(ops, qop, qmul, x);
    else if (r.kind == kKindQ8Ring) pair_qk_q<false>(ops, qop, qmul, x);
    else if (r.kind == kKindF16Ring) pair_qk_16<true>(ops, qop, qmul, x);
    else pair_qk_16<false>(ops, qop, qmul, x);
    if (r.pos0 < lo || r.pos0 + kTile > min(lim, qfirst + 1)) {   // some position hidden from some column
      const int hi = col_ok ? min(lim, qpos_col + 1) : lo;
      const int g4 = lane >> 4;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int pos = r.pos0 + 16 * s + 4 * g4 + rr;
          if (pos < lo || pos >= hi) x[4 * s + rr] = -INFINITY;
        }
    }
    softmax_update(st, x, p);
    if (body || r.kind == kKindQ8Ring) pair_pv_q(st, ops, p);
    else if (r.kind == kKindF16Ring) pair_pv_16<true>(st, ops, p);
    else pair_pv_16<false>(st, ops, p);
  };

  // raw buffer j % 2 decoded into operand buffer j % 2, as the 512 decode threads t of the tile decoders (the
  // combined path of caches without KVarN)
  auto decode_as = [&](int j, int t) {
    if constexpr (!KV) {
      const TileRef r = ref(j);
      Ops& ops = s_ops[j & 1];
      const uint8_t* raw = (const uint8_t*)s_raw[j & 1];
      const bool qb = r.kind == kKindQ;
      const int kcodes = 1024 * (qb ? NK : 8), vcodes = 1024 * (qb ? NV : 8);
      const uint8_t* vscale = raw + r.kbytes + vcodes;
      if (qb) {
        decode_k_tile<NK>(raw, ops, magic, t);
        decode_v_tile<NV>(raw + r.kbytes, vscale, nullptr, ops, magic, t);
      } else {
        decode_k_tile<8>(raw, ops, magic, t);
        decode_v_tile<8>(raw + r.kbytes, vscale, nullptr, ops, magic, t);
      }
      if (t < 32) ((u32x4*)ops.ks)[t] = s_raw[j & 1][kcodes / 16 + t];
    }
  };
  // the bf16 ring's query operand is the bf16 query itself
  auto qop_bf16 = [&]() {
    if (active && g.tail_dtype == 1 && tb < tq) {
      u32x4 qw[8];
      pair_query_words(qrow, col_ok, qw);
#pragma unroll
      for (int b = 0; b < 8; ++b) qop[b] = pair_qop(qw[b], 0, true);
      qmul = a.scale * kLog2e;
    }
  };

  // The pipeline over the quantized tiles [tb, tq), one barrier per tile: in the phase after a barrier, raw buffer
  // (i + 1) % 2 and operand buffer i % 2 hold what the phase before filled, and operand buffer (i + 1) % 2 and raw
  // buffer i % 2 were last read before that barrier. Then the 16-bit ring tiles [tq, te), one tile ahead.
  if (apart) {
    // the quantized tiles in runs of one kind: the body tiles, then the q8_0 ring tiles
    const int tm = min(max(tb, n_body), tq);
    if (wave >= 4) {
      const int t0 = tid - 256;
      u32x4 sk[2] = {};   // KVarN: sigma_K of the lane's 8 channels of K blocks 2c and 2c + 1 (c = wave - 4)
      if (KV && tb < tm) {
#pragma unroll
        for (int h = 0; h < 2; ++h) sk[h] = *(const u32x4*)(sig + 32 * (2 * (wave - 4) + h) + 8 * (lane >> 4));
      }
      if (tb < tm) decode_run_of<NK, NV, KV>(wave - 4, tb, tm, ref, s_ops, magic, lane, sk);
      if (tm < tq) decode_run_of<8, 8, false>(wave - 4, tm, tq, ref, s_ops, magic, lane, sk);
      if (tq < te) {
        constexpr int P16 = 8;   // a 16-bit tile pair: 2048 pieces over 256 threads
        u32x4 r16[P16];
        load_part<P16>(ref(tq), r16, t0, 256);
        for (int i = tq; i < te; ++i) {
          store16_part<P16>(ref(i), s_ops[i & 1], r16, t0, 256);
          if (i + 1 < te) load_part<P16>(ref(i + 1), r16, t0, 256);
          __syncthreads();
        }
      }
      return;
    }
    for (int run = 0; run < 2; ++run) {
      const int r0 = run == 0 ? tb : tm, r1 = run == 0 ? tm : tq;
      if (r0 >= r1) continue;
      __syncthreads();
      for (int i = r0; i < r1; ++i) {
        compute(i, s_ops[i & 1]);
        __syncthreads();
      }
    }
    if (tq < te) {
      qop_bf16();
      for (int i = tq; i < te; ++i) {
        __syncthreads();
        compute(i, s_ops[i & 1]);
      }
    }
  } else if constexpr (!KV) {
    if (tb < tq) {
      stage_part<3>(ref(tb), s_raw[tb & 1], reg, tid, 512);
      if (tb + 1 < tq) load_part<3>(ref(tb + 1), reg, tid, 512);
      __syncthreads();
      decode_as(tb, tid);
      if (tb + 1 < tq) {
        stage_part<3>(ref(tb + 1), s_raw[(tb + 1) & 1], reg, tid, 512);
        if (tb + 2 < tq) load_part<3>(ref(tb + 2), reg, tid, 512);
      }
      __syncthreads();
      for (int i = tb; i < tq; ++i) {
        if (i + 1 < tq) decode_as(i + 1, tid);
        compute(i, s_ops[i & 1]);
        if (i + 2 < tq) {
          stage_part<3>(ref(i + 2), s_raw[i & 1], reg, tid, 512);
          if (i + 3 < tq) load_part<3>(ref(i + 3), reg, tid, 512);
        }
        __syncthreads();
      }
    }
    if (tq < te) {
      qop_bf16();
      u32x4 r16[4];
      load_part<4>(ref(tq), r16, tid, 512);
      for (int i = tq; i < te; ++i) {
        store16_part<4>(ref(i), s_ops[i & 1], r16, tid, 512);
        if (i + 1 < te) load_part<4>(ref(i + 1), r16, tid, 512);
        __syncthreads();
        compute(i, s_ops[i & 1]);
      }
    }
  }
  if (!active) return;

  // ---- outputs: accumulator row j = 4 gq + r holds query 2 wave + (j >= 8), head j & 7
  const float lsum = sum_xor32(sum_xor16(st.l));   // the column's sum over its four lane groups
  const int gq = lane >> 4;
  float hl[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hl[r] = __shfl(lsum, 4 * gq + r);
  const int qo = 2 * wave + (gq >= 2 ? 1 : 0);
  const size_t rec = kPartialHeads * (D + 2);
  if (S.n_splits > 1 && gq == 0) {   // the column's running max and sum
    const int qc = 2 * wave + (m16 >= 8 ? 1 : 0);
    if (qc < nqb) {
      float* pc = a.partials + (((size_t)(row_base + qc) * g.n_kv_heads + head) * a.max_splits + split) * rec;
      pc[hh] = st.m;
      pc[kPartialHeads + hh] = lsum;
    }
  }
  if (qo >= nqb) return;
  // KVarN: the body's V values are still divided by sigma_V per channel (a split of a KVarN cache never mixes body
  // and ring tiles), so a body split's accumulator takes the factor
  const bool sig_v = KV && tb < n_body;
  if (S.n_splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * (gq & 1) + r;
      if (h >= a.group) continue;
      const float inv = hl[r] > 0.0f ? 1.0f / hl[r] : 0.0f;
      float* o = a.out + ((size_t)(row_base + qo) * a.n_q_heads + (size_t)head * a.group + h) * D;
#pragma unroll
      for (int n = 0; n < 16; ++n) o[16 * n + m16] = st.o[n][r] * (sig_v ? h2f(sig[D + 16 * n + m16]) : 1.0f) * inv;
    }
    return;
  }
  float* part = a.partials + (((size_t)(row_base + qo) * g.n_kv_heads + head) * a.max_splits + split) * rec;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * (gq & 1) + r;
#pragma unroll
    for (int n = 0; n < 16; ++n)
      part[2 * kPartialHeads + h * D + 16 * n + m16] = st.o[n][r] * (sig_v ? h2f(sig[D + 16 * n + m16]) : 1.0f);
  }
}

template <int NK, int NV, bool KV>
hipError_t launch_pair_t(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(mq_pair_kernel<NK, NV, KV>, dim3(grid_x), dim3(512), s, e0, e1, a);
}

template <bool KV>
hipError_t launch_pair_dispatch(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nk = a.g.k_bits, nv = a.g.v_bits;
#define KVQ_CASE(K, V) if (nk == K && nv == V) return launch_pair_t<K, V, KV>(a, grid_x, s, e0, e1);
#define KVQ_ROW(K) KVQ_CASE(K, 2) KVQ_CASE(K, 3) KVQ_CASE(K, 4) KVQ_CASE(K, 5) KVQ_CASE(K, 6) KVQ_CASE(K, 7) KVQ_CASE(K, 8)
  KVQ_ROW(2) KVQ_ROW(3) KVQ_ROW(4) KVQ_ROW(5) KVQ_ROW(6) KVQ_ROW(7) KVQ_ROW(8)
#undef KVQ_ROW
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kvq
