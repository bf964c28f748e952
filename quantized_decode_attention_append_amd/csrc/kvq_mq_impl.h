// Multi-query attention over the quantized cache: blocks of up to 8 consecutive query positions of a sequence
// attend causally to the cache, each K / V tile read from HBM and decoded once for all of them. It also serves
// single-query decode of caches with qN_1 bodies (a scale and a minimum per block, BeeLlama page q2_1 .. q6_1)
// and with token-axis K (KIVI-style per-channel K blocks, Qwen3.8-27B page, reader comment). It serves the
// verification of drafted tokens (Qwen3.8-27B page, decode-speed paragraph: the engine drafts up to 7 tokens per
// step with MTP heads) and chunked prefill over the quantized cache (the KVarN benchmark page and the
// Qwen3.8-27B page measure prompt processing per cache type).
//
// A work-group of 8 waves takes one query block of one KV head over a range of the block's prefix tiles (the
// qN_0 body tiles, then the ring tiles). Per 32-position tile:
// * the work-group loads the raw tile once (every thread one to four 16-byte pieces, one tile ahead in
//   registers) and decodes it cooperatively into MFMA operands in LDS, in the operand order of the decode
//   kernel: K codes as exact fp16 integers (the "1024 + value" form) with the tile's fp16 K scales, and each V
//   code times its block scale as an fp16 pair, the rounded product and the (exact) remainder; bf16 / f16 ring
//   tiles are stored in that order already and are copied as they are;
// * wave w then computes query w of the block on its own: QK on MFMA (8 heads of the group as hi / lo fp16
//   columns of the exponent-shifted query), the per-(position, block) K scale in fp32, its own causal mask,
//   online softmax, and P.V on MFMA with A = P split into hi / lo fp16 rows, against both V parts.
// The operands are double-buffered, so a tile costs two work-group barriers. Each wave writes its query's
// partial (max, sum, output) record; with one split per block it writes the normalized output instead.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"
#include "kvq_mfma.h"

namespace kvq {
namespace {

constexpr int kMqWaves = 8;
constexpr int kRawChunks = 2 * 32 * 288 / 16;   // 16-byte pieces of the largest quantized tile pair (q8_1 K + V)

template <bool VAR>
struct MqOpsT {                // one tile's MFMA operands in LDS (VAR: with the qN_1 / token-axis K operands)
  u32x4 k[2 * 8 * 64];         // K operands [subtile][block][lane]: 8 codes (or 16-bit values) per lane
  u32x4 v[16 * 64];            // V operands [n-tile][lane]: code x scale (+ offset), fp16 rounded (or 16-bit values)
  u32x4 vl[16 * 64];           // V operands, the remainders, fp16
  uint16_t ks[8 * 32];         // K scales [block][position]
  u32x4 kmin[VAR ? 2 * 64 : 1];     // qN_1 K: A operand of the offset term [subtile][lane] (rows: positions; k 0-7:
                                    // the blocks' offsets, fp16 hi parts; k 8-15: lo parts; k 16-31: zero)
  u32x4 kl[VAR ? 2 * 8 * 64 : 1];   // token-axis K: the remainders of the scaled K values (k holds the rounded ones)
};

enum { kKindQ = 0, kKindQ8Ring = 1, kKindBf16Ring = 2, kKindF16Ring = 3 };

// Where one tile of an entry's list lives, and how it is stored.
struct TileRef {
  const uint8_t* k;
  const uint8_t* v;
  int kbytes, vbytes;
  int kind;       // kKind*
  int pos0;       // first position of the tile (its position tile x 32)
};

// ---------------------------------------------------------------------------- cooperative tile decode

// Lane run of one plane of a K subtile in the raw tile: [chunk][lane][unit], unit = min(16, 8w) bytes.
template <int W>
__device__ inline void raw_k_run(const uint8_t* raw, int base, int lane, uint32_t* dst) {
  constexpr int lb = 8 * W;
  constexpr int unit = lb < 16 ? lb : 16;
#pragma unroll
  for (int u = 0; u < lb / unit; ++u) {
    if constexpr (unit == 16) {
      const u32x4 x = *(const u32x4*)(raw + base + (u * 64 + lane) * 16);
      dst[4 * u] = x[0]; dst[4 * u + 1] = x[1]; dst[4 * u + 2] = x[2]; dst[4 * u + 3] = x[3];
    } else {
      const u32x2 x = *(const u32x2*)(raw + base + lane * unit);
      dst[2 * u] = x[0]; dst[2 * u + 1] = x[1];
    }
  }
}

// Lane run of one plane of a V tile in the raw tile: 16 pieces of w bits x 8, [chunk][lane][16 B].
template <int W>
__device__ inline void raw_v_run(const uint8_t* raw, int base, int lane, uint32_t* dst) {
  constexpr int lb = 16 * W;
#pragma unroll
  for (int u = 0; u < lb / 16; ++u) {
    const u32x4 x = *(const u32x4*)(raw + base + (u * 64 + lane) * 16);
    dst[4 * u] = x[0]; dst[4 * u + 1] = x[1]; dst[4 * u + 2] = x[2]; dst[4 * u + 3] = x[3];
  }
}

template <int N, int I0>
__device__ inline void k_two_pieces(const uint32_t* r0, const uint32_t* r1, const uint32_t* r2, uint32_t magic,
                                    u32x4* dst) {
  dst[0] = __builtin_bit_cast(u32x4, decode_run_piece<N, I0>(r0, r1, r2, magic));
  dst[64] = __builtin_bit_cast(u32x4, decode_run_piece<N, I0 + 1>(r0, r1, r2, magic));
}

// K operands of one tile, as 512 threads t (the work-group's threads, or its last 256 taking two t each): the
// wave w = t / 64 decodes blocks 2(w % 4) and 2(w % 4) + 1 of subtile w / 4 (the block pair is uniform across the
// wave, so the wave runs one of the four decode variants), thread t lane t % 64.
template <int N, class Ops>
__device__ inline void decode_k_tile(const uint8_t* raw, Ops& ops, uint32_t magic, int t) {
  constexpr int w0 = Planes<N>::w[0], w1 = Planes<N>::w[1], w2 = Planes<N>::w[2];
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int s = wv >> 2, bp = wv & 3, lane = t & 63;
  uint32_t r0[2 * w0], r1[w1 ? 2 * w1 : 1], r2[w2 ? 2 * w2 : 1];
  const int sub = 512 * N * s;
  raw_k_run<w0>(raw, sub, lane, r0);
  if constexpr (w1 > 0) raw_k_run<w1>(raw, sub + 512 * w0, lane, r1);
  if constexpr (w2 > 0) raw_k_run<w2>(raw, sub + 512 * (w0 + w1), lane, r2);
  u32x4* dst = ops.k + (s * 8 + 2 * bp) * 64 + lane;
  switch (bp) {
    case 0: k_two_pieces<N, 0>(r0, r1, r2, magic, dst); break;
    case 1: k_two_pieces<N, 2>(r0, r1, r2, magic, dst); break;
    case 2: k_two_pieces<N, 4>(r0, r1, r2, magic, dst); break;
    default: k_two_pieces<N, 6>(r0, r1, r2, magic, dst); break;
  }
}

// A V piece (8 exact fp16 codes, positions in operand order) times the scales of its positions: the fp16
// rounded products and their remainders (each remainder exact: a product of an 8-bit code and an fp16 scale
// has at most 19 significant bits).
__device__ inline void scale_v_piece(half8 c, const uint32_t* dv, u32x4& hi, u32x4& lo) {
  const u32x4 r = __builtin_bit_cast(u32x4, c);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const half2v h = as_h2(r[k]) * as_h2(dv[k]);
    hi[k] = as_u(h);
    lo[k] = as_u(__builtin_elementwise_fma(as_h2(r[k]), as_h2(dv[k]), -h));
  }
}

// qN_1: a V piece's values code x scale + offset (offset = minimum + 2^(N-1) x scale: the codes are decoded
// signed, c = u - 2^(N-1)) in fp32, as fp16 rounded values and remainders (to ~22 bits).
__device__ inline void scale_v_piece_min(half8 c, const uint32_t* dv, const float* off, u32x4& hi, u32x4& lo) {
  const u32x4 r = __builtin_bit_cast(u32x4, c);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const half2v cv = as_h2(r[k]), d = as_h2(dv[k]);
    const float x0 = fmaf((float)cv[0], (float)d[0], off[2 * k]);
    const float x1 = fmaf((float)cv[1], (float)d[1], off[2 * k + 1]);
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    hi[k] = as_u(half2v{h0, h1});
    lo[k] = as_u(half2v{(_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)});
  }
}

// V operands of one tile, as 512 threads t: thread t decodes n-tiles 2(t / 64) and 2(t / 64) + 1 (block t / 64)
// of lane t % 64; vscale: the tile's V scales [block][position]; vmin: a qN_1 tile's minima [block][position],
// else null.
template <int N, class Ops>
__device__ inline void decode_v_tile(const uint8_t* raw, const uint8_t* vscale, const uint8_t* vmin, Ops& ops,
                                     uint32_t magic, int t) {
  constexpr int w0 = Planes<N>::w[0], w1 = Planes<N>::w[1], w2 = Planes<N>::w[2];
  const int lane = t & 63, np = __builtin_amdgcn_readfirstlane(t >> 6), g = lane >> 4;
  uint32_t r0[4 * w0], r1[w1 ? 4 * w1 : 1], r2[w2 ? 4 * w2 : 1];
  raw_v_run<w0>(raw, 0, lane, r0);
  if constexpr (w1 > 0) raw_v_run<w1>(raw, 1024 * w0, lane, r1);
  if constexpr (w2 > 0) raw_v_run<w2>(raw, 1024 * (w0 + w1), lane, r2);
  // the scales of operand rows 8g..8g+7: positions 4g..4g+3 and 16+4g..16+4g+3 of block np
  const u32x2 d0 = *(const u32x2*)(vscale + 2 * (np * 32 + 4 * g));
  const u32x2 d1 = *(const u32x2*)(vscale + 2 * (np * 32 + 16 + 4 * g));
  const uint32_t dv[4] = {d0[0], d0[1], d1[0], d1[1]};
  const int o = 2 * np * 64 + lane;
  if (vmin) {
    const u32x2 m0 = *(const u32x2*)(vmin + 2 * (np * 32 + 4 * g));
    const u32x2 m1 = *(const u32x2*)(vmin + 2 * (np * 32 + 16 + 4 * g));
    const uint32_t mw[4] = {m0[0], m0[1], m1[0], m1[1]};
    float off[8];
    constexpr float bias = (float)(1 << (N - 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      off[2 * k] = fmaf(bias, lo_h(dv[k]), lo_h(mw[k]));
      off[2 * k + 1] = fmaf(bias, hi_h(dv[k]), hi_h(mw[k]));
    }
#define KVQ_VPM(P)                                                                                                 \
  case P:                                                                                                          \
    scale_v_piece_min(decode_run_piece<N, 2 * P>(r0, r1, r2, magic), dv, off, ops.v[o], ops.vl[o]);               \
    scale_v_piece_min(decode_run_piece<N, 2 * P + 1>(r0, r1, r2, magic), dv, off, ops.v[o + 64], ops.vl[o + 64]); \
    break;
    switch (np) { KVQ_VPM(0) KVQ_VPM(1) KVQ_VPM(2) KVQ_VPM(3) KVQ_VPM(4) KVQ_VPM(5) KVQ_VPM(6) default: KVQ_VPM(7) }
#undef KVQ_VPM
    return;
  }
#define KVQ_VP(P)                                                                                        \
  case P:                                                                                                \
    scale_v_piece(decode_run_piece<N, 2 * P>(r0, r1, r2, magic), dv, ops.v[o], ops.vl[o]);                \
    scale_v_piece(decode_run_piece<N, 2 * P + 1>(r0, r1, r2, magic), dv, ops.v[o + 64], ops.vl[o + 64]);  \
    break;
  switch (np) { KVQ_VP(0) KVQ_VP(1) KVQ_VP(2) KVQ_VP(3) KVQ_VP(4) KVQ_VP(5) KVQ_VP(6) default: KVQ_VP(7) }
#undef KVQ_VP
}

// Token-axis K operands of one tile (a block is the 32 positions of one channel: one scale, and for qN_1 one
// minimum, per channel): thread t as in decode_k_tile, its 16 channels' values code x scale (+ offset) as fp16
// rounded values and remainders. kscale / kmin: the tile's scales and minima [channel] (kmin null for qN_0).
template <int N, class Ops>
__device__ inline void decode_k_tile_tok(const uint8_t* raw, const uint8_t* kscale, const uint8_t* kmin, Ops& ops,
                                         uint32_t magic) {
  constexpr int w0 = Planes<N>::w[0], w1 = Planes<N>::w[1], w2 = Planes<N>::w[2];
  const int t = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int s = wv >> 2, bp = wv & 3, lane = t & 63, g = lane >> 4;
  uint32_t r0[2 * w0], r1[w1 ? 2 * w1 : 1], r2[w2 ? 2 * w2 : 1];
  const int sub = 512 * N * s;
  raw_k_run<w0>(raw, sub, lane, r0);
  if constexpr (w1 > 0) raw_k_run<w1>(raw, sub + 512 * w0, lane, r1);
  if constexpr (w2 > 0) raw_k_run<w2>(raw, sub + 512 * (w0 + w1), lane, r2);
  half8 c[2];
  switch (bp) {
    case 0: c[0] = decode_run_piece<N, 0>(r0, r1, r2, magic); c[1] = decode_run_piece<N, 1>(r0, r1, r2, magic); break;
    case 1: c[0] = decode_run_piece<N, 2>(r0, r1, r2, magic); c[1] = decode_run_piece<N, 3>(r0, r1, r2, magic); break;
    case 2: c[0] = decode_run_piece<N, 4>(r0, r1, r2, magic); c[1] = decode_run_piece<N, 5>(r0, r1, r2, magic); break;
    default: c[0] = decode_run_piece<N, 6>(r0, r1, r2, magic); c[1] = decode_run_piece<N, 7>(r0, r1, r2, magic); break;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = 2 * bp + h;
    const int ch0 = 32 * b + 8 * g;   // the piece's 8 channels
    const u32x4 dw = *(const u32x4*)(kscale + 2 * ch0);
    const u32x4 cw = __builtin_bit_cast(u32x4, c[h]);
    u32x4 hi, lo;
    if (kmin) {
      const u32x4 mw = *(const u32x4*)(kmin + 2 * ch0);
      constexpr float bias = (float)(1 << (N - 1));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const half2v cv = as_h2(cw[k]), d = as_h2(dw[k]), m = as_h2(mw[k]);
        const float x0 = fmaf((float)cv[0], (float)d[0], fmaf(bias, (float)d[0], (float)m[0]));
        const float x1 = fmaf((float)cv[1], (float)d[1], fmaf(bias, (float)d[1], (float)m[1]));
        const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
        hi[k] = as_u(half2v{h0, h1});
        lo[k] = as_u(half2v{(_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)});
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // code x scale has at most 19 significant bits: value + exact remainder
        const half2v pr = as_h2(cw[k]) * as_h2(dw[k]);
        hi[k] = as_u(pr);
        lo[k] = as_u(__builtin_elementwise_fma(as_h2(cw[k]), as_h2(dw[k]), -pr));
      }
    }
    const int o = (s * 8 + b) * 64 + lane;
    ops.k[o] = hi;
    ops.kl[o] = lo;
  }
}

// QK of a token-axis K tile: the scaled values and their remainders against the query operand, all blocks into one
// accumulator per subtile (the scales are already in the operands).
template <class Ops>
__device__ inline void mq_qk_tok(const Ops& ops, const half8* qop, float qmul, float* x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    floatx4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.k[(s * 8 + b) * 64 + lane]), qop[b], c0,
                                                  0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.kl[(s * 8 + b) * 64 + lane]), qop[b], c1,
                                                  0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = c0[r] + c1[r];
      x[4 * s + r] = (v + dpp_ror8(v)) * qmul;
    }
  }
}

// qN_1 K: the A operand of the offset term for subtile s, lane (g, m16): row = position 16s + m16; g = 0 holds
// the fp16 hi parts of the 8 blocks' offsets (minimum + 2^(N-1) x scale, fp32), g = 1 the lo parts, g = 2, 3 zero.
// kscale: the tile's K scales [block][position]; kmin: its minima [position][block]. Threads 0-127.
template <int N, class Ops>
__device__ inline void kmin_operand(const uint8_t* kscale, const uint8_t* kmin, Ops& ops) {
  const int t = threadIdx.x;
  const int s = t >> 6, lane = t & 63, g = lane >> 4;
  const int pos = 16 * s + (lane & 15);
  u32x4 out = {0u, 0u, 0u, 0u};
  if (g < 2) {
    const u32x4 mw = *(const u32x4*)(kmin + 16 * pos);
    constexpr float bias = (float)(1 << (N - 1));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float d0 = h2f(((const uint16_t*)kscale)[(2 * k) * 32 + pos]);
      const float d1 = h2f(((const uint16_t*)kscale)[(2 * k + 1) * 32 + pos]);
      const float o0 = fmaf(bias, d0, lo_h(mw[k])), o1 = fmaf(bias, d1, hi_h(mw[k]));
      const _Float16 h0 = (_Float16)o0, h1 = (_Float16)o1;
      out[k] = g == 0 ? as_u(half2v{h0, h1})
                      : as_u(half2v{(_Float16)(o0 - (float)h0), (_Float16)(o1 - (float)h1)});
    }
  }
  ops.kmin[s * 64 + lane] = out;
}

// ---------------------------------------------------------------------------- per-wave compute

// QK of a qN_0 (or q8_0 ring) tile for this wave's query: block by block one MFMA per 16-row subtile, the K scale
// of each (position, block) applied to the fp32 result. x[4s + r]: position 16s + 4g + r.
template <bool VAR, class Ops>
__device__ inline void mq_qk_q(const Ops& ops, const half8* qop, float qmul, float* x, const u32x4* qsum) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float sc[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (VAR && qsum) {   // qN_1: sum over blocks of offset x the query's block sum, one MFMA per subtile
    const half8 b = __builtin_bit_cast(half8, *qsum);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.kmin[s * 64 + lane]), b,
                                                               floatx4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[s][r] = c[r];
    }
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const floatx4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.k[b * 64 + lane]), qop[b],
                                                              floatx4{0, 0, 0, 0}, 0, 0, 0);
    const floatx4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.k[(8 + b) * 64 + lane]),
                                                              qop[b], floatx4{0, 0, 0, 0}, 0, 0, 0);
    const u32x2 d0 = *(const u32x2*)(ops.ks + b * 32 + 4 * g);
    const u32x2 d1 = *(const u32x2*)(ops.ks + b * 32 + 16 + 4 * g);
    sc[0][0] = fmaf(c0[0], lo_h(d0[0]), sc[0][0]);
    sc[0][1] = fmaf(c0[1], hi_h(d0[0]), sc[0][1]);
    sc[0][2] = fmaf(c0[2], lo_h(d0[1]), sc[0][2]);
    sc[0][3] = fmaf(c0[3], hi_h(d0[1]), sc[0][3]);
    sc[1][0] = fmaf(c1[0], lo_h(d1[0]), sc[1][0]);
    sc[1][1] = fmaf(c1[1], hi_h(d1[0]), sc[1][1]);
    sc[1][2] = fmaf(c1[2], lo_h(d1[1]), sc[1][2]);
    sc[1][3] = fmaf(c1[3], hi_h(d1[1]), sc[1][3]);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * s + r] = (sc[s][r] + dpp_ror8(sc[s][r])) * qmul;
}

// P.V of a qN_0 (or q8_0 ring) tile: A = P as fp16 hi (rows 0-7) and lo (rows 8-15) parts, against the scaled
// V values and their remainders, so the four partial products sum to P x code x scale.
template <class Ops>
__device__ inline void mq_pv_q(WaveState& st, const Ops& ops, const float* p, bool lo_lane) {
  const int lane = threadIdx.x & 63;
  const float kf = lo_lane ? 1.0f : 0.0f;
  half8 a;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)p[i];
    a[i] = (_Float16)fmaf(-kf, (float)h, p[i]);
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, ops.v[n * 64 + lane]), st.o[n], 0, 0,
                                                     0);
    st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, ops.vl[n * 64 + lane]), st.o[n], 0,
                                                     0, 0);
  }
}

// QK and P.V of a 16-bit ring tile (values stored as they are: bf16 with bf16 MFMA, f16 with fp16 MFMA).
template <bool F16, class Ops>
__device__ inline void mq_qk_16(const Ops& ops, const u32x4* qop, float qmul, float* x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    floatx4 c = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if constexpr (F16)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ops.k[(s * 8 + b) * 64 + lane]),
                                                   __builtin_bit_cast(half8, qop[b]), c, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ops.k[(s * 8 + b) * 64 + lane]),
                                                    __builtin_bit_cast(bf16x8, qop[b]), c, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * s + r] = (F16 ? c[r] + dpp_ror8(c[r]) : c[r]) * qmul;
  }
}

template <bool F16, class Ops>
__device__ inline void mq_pv_16(WaveState& st, const Ops& ops, const float* p, bool lo_lane) {
  const int lane = threadIdx.x & 63;
  const float kf = lo_lane ? 1.0f : 0.0f;
  if constexpr (F16) {
    half8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const _Float16 h = (_Float16)p[i];
      a[i] = (_Float16)fmaf(-kf, (float)h, p[i]);
    }
#pragma unroll
    for (int n = 0; n < 16; ++n)
      st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, ops.v[n * 64 + lane]), st.o[n], 0,
                                                       0, 0);
  } else {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)p[i];
      a[i] = (__bf16)fmaf(-kf, (float)h, p[i]);
    }
#pragma unroll
    for (int n = 0; n < 16; ++n)
      st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, ops.v[n * 64 + lane]), st.o[n],
                                                        0, 0, 0);
  }
}

// ---------------------------------------------------------------------------- the kernel

__device__ __attribute__((always_inline)) inline TileRef tile_ref(const MqArgs& a, const MqSeq& S, int head, int i, int n_body) {
  const Geometry& g = a.g;
  const uint8_t* slab = g.arena + S.slab;
  TileRef r;
  if (i < n_body) {
    r.k = slab + g.k_body + ((size_t)head * (g.cap32 / kTile) + i) * g.tile_k;
    r.v = slab + g.v_body + ((size_t)head * (g.cap32 / kTile) + i) * g.tile_v;
    r.kbytes = g.tile_k;
    r.vbytes = g.tile_v;
    r.kind = kKindQ;
    r.pos0 = i * kTile;
  } else {
    const int t = S.body_len / kTile + (i - n_body);
    const int R = g.ring_slots;
    const size_t rt = (size_t)head * (R / kTile) + ((t * kTile) % R) / kTile;
    r.k = slab + g.k_ring + rt * g.ring_tile_k;
    r.v = slab + g.v_ring + rt * g.ring_tile_v;
    r.kbytes = g.ring_tile_k;
    r.vbytes = g.ring_tile_v;
    r.kind = g.tail_dtype == 2 ? kKindQ8Ring : g.tail_dtype == 1 ? kKindBf16Ring : kKindF16Ring;
    r.pos0 = t * kTile;
  }
  return r;
}

// The 16-byte pieces of a tile that thread t loads: piece c = t + 512 j of [K tile][V tile].
constexpr int kMaxPieces = 4;   // a 16-bit ring tile pair: 32 KiB = 4 pieces per thread
__device__ inline void load_pieces(const TileRef& r, u32x4* reg) {
  const int nk = r.kbytes / 16, nv = r.vbytes / 16;
#pragma unroll
  for (int j = 0; j < kMaxPieces; ++j) {
    const int c = threadIdx.x + 512 * j;
    if (c < nk) reg[j] = __builtin_nontemporal_load((const u32x4*)r.k + c);
    else if (c < nk + nv) reg[j] = __builtin_nontemporal_load((const u32x4*)r.v + (c - nk));
  }
}

// The lane's query words: channels 32b + 8g .. 32b + 8g + 7 of block b (g = lane / 16) of its head, bf16, and the
// same channels of `sig` (KVarN sigma of K; fp16 1 without it). The lanes of a wave together hold every head of the
// group, so one batch of loads serves the exponent shift and the operand.
__device__ inline void query_words(const uint16_t* qrow, const uint16_t* sig, u32x4* qw, u32x4* sw) {
  const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    qw[b] = *(const u32x4*)(qrow + 32 * b + 8 * gq);
    sw[b] = sig ? *(const u32x4*)(sig + 32 * b + 8 * gq) : u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  }
}

// Exponent shift of a query: its |q sigma| maximum over the group's heads brought below 2^9.
__device__ inline int query_shift(const u32x4* qw, const u32x4* sw, bool head_ok) {
  float amax = 0.0f;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      amax = fmaxf(amax, fabsf(__uint_as_float(qw[b][k] << 16) * lo_h(sw[b][k])));
      amax = fmaxf(amax, fabsf(__uint_as_float(qw[b][k] & 0xFFFF0000u) * hi_h(sw[b][k])));
    }
  if (!head_ok) amax = 0.0f;
  amax = wave_max_16_32(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  return amax > 0.0f ? ilogbf(amax) - 8 : 0;
}

// Hi / lo fp16 query operand of one block (columns 0-7: hi parts of the group's heads, 8-15: lo parts) from the
// lane's words: the query times `sig` and 2^-e.
// Returns the sum of this lane's 8 (exact) operand values, for the block sums of a qN_1 K.
__device__ inline float build_qop_f16(const u32x4& qw, const u32x4& sw, int e, bool head_ok, bool lo_lane,
                                      half8& out) {
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = ldexpf(__uint_as_float(qw[k] << 16) * lo_h(sw[k]), -e);          // exact: 8 + 11 bits
    const float x1 = ldexpf(__uint_as_float(qw[k] & 0xFFFF0000u) * hi_h(sw[k]), -e);
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
    out[2 * k] = head_ok ? (lo_lane ? l0 : h0) : (_Float16)0.0f;
    out[2 * k + 1] = head_ok ? (lo_lane ? l1 : h1) : (_Float16)0.0f;
    sum += x0 + x1;
  }
  return head_ok ? sum : 0.0f;
}

// VAR: the instantiation that reads qN_1 bodies and token-axis K (the plain one compiles those paths out)
template <int NK, int NV, bool VAR>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mq_kernel(MqArgs a) {
  constexpr int D = 256;
  __shared__ MqOpsT<VAR> s_ops[2];
  __shared__ u32x4 s_raw[kRawChunks];
  __shared__ u32x4 s_qsum[VAR ? kMqWaves * 64 : 1];   // qN_1 K: each wave's B operand of the offset term
  const Geometry& g = a.g;
  const bool k_min = VAR && g.k_min, v_min = VAR && g.v_min, k_axis = VAR && g.k_axis;
  // work-group -> (sequence, query block, KV head, split)
  int si = 0;
  while (si + 1 < a.n_seqs && a.seqs[si + 1].wg_begin <= (int)blockIdx.x) ++si;
  const MqSeq& S = a.seqs[si];
  int rem = blockIdx.x - S.wg_begin;
  const int split = rem % S.n_splits;
  rem /= S.n_splits;
  const int head = rem % g.n_kv_heads;
  const int qblk = rem / g.n_kv_heads;
  const int qb0 = S.q0 + kMqWaves * qblk;                // first query position of the block
  const int nqb = min(kMqWaves, S.nq - kMqWaves * qblk);
  const int end = qb0 + nqb;                             // the block attends to positions [0, end)
  const int blen = min(S.body_len, end);
  const int n_body = (blen + kTile - 1) / kTile;
  const int n_ring = end > S.body_len ? (end + kTile - 1) / kTile - S.body_len / kTile : 0;
  const int n_tiles = n_body + n_ring;
  // this split's tiles [tb, te): with n_ring_splits == 0 the splits share the whole list (body tiles, then ring
  // tiles); otherwise the first n_splits - n_ring_splits share the body tiles and the rest the ring tiles
  int tb, te;
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

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m16 = lane & 15;
  const int hh = m16 & 7;
  const bool lo_lane = m16 >= 8;
  const bool head_ok = hh < a.group;
  const bool active = wave < nqb;
  const int qpos = qb0 + wave;                            // this wave's query position (when active)
  const int row = S.row0 + kMqWaves * qblk + wave;
  const uint16_t* qgroup = a.q + ((size_t)row * a.n_q_heads + (size_t)head * a.group) * D;
  const uint16_t* qrow = qgroup + (size_t)(head_ok ? hh : 0) * D;
  const uint16_t* sig = g.kvarn ? (const uint16_t*)(g.arena + S.slab + g.sigma) + (size_t)head * 2 * D : nullptr;

  // this wave's query operand, built for the kind of tile at hand (a split switches at most once, from the body
  // tiles to the ring tiles): the body's is the query times sigma_K (KVarN), exponent-shifted, as fp16 hi / lo
  // columns; the q8_0 ring's the same without sigma; the f16 ring's hi / lo fp16 unshifted; the bf16 ring's the
  // bf16 query itself (columns 8-15 repeat heads 0-7, so the lo-part lanes see the same scores)
  half8 qop[8];
  float qmul = 0.0f;
  int qop_kind = -1;
  auto build_qop = [&](int kind) {
    if (kind == kKindQ || kind == kKindQ8Ring) {
      const uint16_t* sg = kind == kKindQ ? sig : nullptr;
      u32x4 qw[8], sw[8];
      query_words(qrow, sg, qw, sw);
      const int e = query_shift(qw, sw, head_ok);
      float bsum[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) bsum[b] = build_qop_f16(qw[b], sw[b], e, head_ok, lo_lane, qop[b]);
      qmul = a.scale * kLog2e * ldexpf(1.0f, e);
      if (kind == kKindQ && k_min && !k_axis) {
        // qN_1 K: the B operand of the offset term, lane (g, m16): k = 8g + b (g = 0, 1) is the block-b sum of
        // the operand values of head m16 & 7 (over the 4 lane groups), its fp16 hi part in columns 0-7 and its
        // lo part in columns 8-15; g = 2, 3 zero
        half8 qs;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const float t = sum_xor32(sum_xor16(bsum[b]));
          const _Float16 h = (_Float16)t;
          const _Float16 part = lo_lane ? (_Float16)(t - (float)h) : h;
          qs[b] = (lane >> 4) < 2 ? part : (_Float16)0.0f;
        }
        s_qsum[wave * 64 + lane] = __builtin_bit_cast(u32x4, qs);
      }
    } else if (kind == kKindF16Ring) {
      u32x4 qw[8], sw[8];
      query_words(qrow, nullptr, qw, sw);
#pragma unroll
      for (int b = 0; b < 8; ++b) build_qop_f16(qw[b], sw[b], 0, head_ok, lo_lane, qop[b]);
      qmul = a.scale * kLog2e;
    } else {
      const int gq = lane >> 4;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        u32x4 w = *(const u32x4*)(qrow + 32 * b + 8 * gq);
        if (!head_ok) w = u32x4{0u, 0u, 0u, 0u};
        qop[b] = __builtin_bit_cast(half8, w);
      }
      qmul = a.scale * kLog2e;
    }
    qop_kind = kind;
  };
  const bool has_body = tb < n_body;

  WaveState st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int n = 0; n < 16; ++n) st.o[n] = floatx4{0, 0, 0, 0};
  uint32_t magic = kMagic;
  asm volatile("" : "+v"(magic));

  u32x4 reg[kMaxPieces];
  TileRef cur;
  if (tb < te) {
    cur = tile_ref(a, S, head, tb, n_body);
    load_pieces(cur, reg);
  }
  int buf = 0;
  for (int i = tb; i < te; ++i, buf ^= 1) {
    MqOpsT<VAR>& ops = s_ops[buf];
    const TileRef r = cur;
    const int nk = r.kbytes / 16, nv = r.vbytes / 16;
    const bool raw16 = r.kind == kKindBf16Ring || r.kind == kKindF16Ring;
    // this tile's pieces into LDS: 16-bit ring tiles straight into the operand buffers, the others into the raw
    // buffer for the decode below
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      const int c = tid + 512 * j;
      if (c < nk + nv) {
        if (raw16) {
          if (c < nk) ops.k[c] = reg[j];
          else ops.v[c - nk] = reg[j];
        } else {
          s_raw[c] = reg[j];
        }
      }
    }
    // the next tile's loads go out now and are in flight during this tile's decode and compute
    if (i + 1 < te) {
      cur = tile_ref(a, S, head, i + 1, n_body);
      load_pieces(cur, reg);
    }
    __syncthreads();
    if (!raw16) {
      const uint8_t* raw = (const uint8_t*)s_raw;
      // a quantized tile: the codes (1024 N bytes), the scales [block][position], then for a qN_1 body the minima
      const bool qb = r.kind == kKindQ;
      const int kcodes = 1024 * (qb ? NK : 8), vcodes = 1024 * (qb ? NV : 8);
      const uint8_t* vscale = raw + r.kbytes + vcodes;
      if (qb) {
        if constexpr (VAR) {
          if (k_axis) {
            decode_k_tile_tok<NK>(raw, raw + kcodes, k_min ? raw + kcodes + 512 : nullptr, ops, magic);
          } else {
            decode_k_tile<NK>(raw, ops, magic, tid);
            if (k_min && tid < 128) kmin_operand<NK>(raw + kcodes, raw + kcodes + 512, ops);
          }
        } else {
          decode_k_tile<NK>(raw, ops, magic, tid);
        }
        decode_v_tile<NV>(raw + r.kbytes, vscale, v_min ? vscale + 512 : nullptr, ops, magic, tid);
      } else {
        decode_k_tile<8>(raw, ops, magic, tid);
        decode_v_tile<8>(raw + r.kbytes, vscale, nullptr, ops, magic, tid);
      }
      if (tid < 32) ((u32x4*)ops.ks)[tid] = s_raw[kcodes / 16 + tid];
      __syncthreads();
    }
    // this wave's query over the tile: positions [lo, hi) of the tile's segment, causally up to qpos
    if (active) {
      const bool body = r.kind == kKindQ;
      const int lo = body ? 0 : S.body_len;
      const int hi = min(body ? blen : end, qpos + 1);
      if (r.pos0 < hi && r.pos0 + kTile > lo) {
        if (r.kind != qop_kind) build_qop(r.kind);
        float x[8], p[8];
        if (VAR && body && k_axis) {
          if constexpr (VAR) mq_qk_tok(ops, qop, qmul, x);
        } else if (body || r.kind == kKindQ8Ring) {
          mq_qk_q<VAR>(ops, qop, qmul, x, VAR && body && k_min ? &s_qsum[wave * 64 + lane] : nullptr);
        }
        else if (r.kind == kKindF16Ring) mq_qk_16<true>(ops, (const u32x4*)qop, qmul, x);
        else mq_qk_16<false>(ops, (const u32x4*)qop, qmul, x);
        const int g4 = lane >> 4;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int pos = r.pos0 + 16 * s + 4 * g4 + rr;
            if (pos < lo || pos >= hi) x[4 * s + rr] = -INFINITY;
          }
        softmax_update(st, x, p);
        if (body || r.kind == kKindQ8Ring) mq_pv_q(st, ops, p, lo_lane);
        else if (r.kind == kKindF16Ring) mq_pv_16<true>(st, ops, p, lo_lane);
        else mq_pv_16<false>(st, ops, p, lo_lane);
      }
    }
  }
  if (!active) return;

  // ---- this wave's query: l over the lanes of a head, o = hi rows + lo rows
  const float lsum = sum_xor32(sum_xor16(lo_lane ? 0.0f : st.l));
#pragma unroll
  for (int n = 0; n < 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[n][r] = sum_xor32(st.o[n][r]);
  const int gq = lane >> 4;
  // the sums of heads 4 gq + r (rows of the first two row groups) from lanes 4 gq + r
  float hl[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) hl[r] = __shfl(lsum, 4 * gq + r);
  if (gq >= 2) return;
  // KVarN: the body's V values are still divided by sigma_V per channel; a split of a KVarN cache never mixes body
  // and ring tiles (the host plans separate splits), so the factor applies to the whole accumulator
  const bool sig_v = g.kvarn && has_body;
  if (S.n_splits == 1) {
    // the whole prefix in this work-group: the normalized output
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * gq + r;
      if (h >= a.group) continue;
      const float inv = hl[r] > 0.0f ? 1.0f / hl[r] : 0.0f;
      float* o = a.out + ((size_t)row * a.n_q_heads + (size_t)head * a.group + h) * D;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int c = 16 * n + m16;
        const float vs = sig_v ? h2f(sig[D + c]) : 1.0f;
        o[c] = st.o[n][r] * vs * inv;
      }
    }
    return;
  }
  float* part = a.partials + (((size_t)row * g.n_kv_heads + head) * a.max_splits + split) * (kPartialHeads * (D + 2));
  if (gq == 0 && m16 < 8) {
    part[m16] = st.m;   // lanes 0-7: heads 0-7
    part[kPartialHeads + m16] = lsum;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * gq + r;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int c = 16 * n + m16;
      const float vs = sig_v ? h2f(sig[D + c]) : 1.0f;
      part[2 * kPartialHeads + h * D + c] = st.o[n][r] * vs;
    }
  }
}

// Merge of the split partials of every query row: one work-group per (row, KV head, query head), 16 groups of 64
// threads, thread t of a group owning channels 4t .. 4t + 3 of a strided share of the splits (online log-sum-exp,
// exp2 domain); then the 16 groups are merged: out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
__global__ __launch_bounds__(1024) void mq_combine_kernel(MqArgs a) {
  constexpr int D = 256;
  constexpr size_t rec = kPartialHeads * (D + 2);
  __shared__ float s_m[16], s_l[16];
  __shared__ floatx4 s_o[16][64];
  const int hk = a.g.n_kv_heads;
  const int row = blockIdx.x / hk;
  const int head = blockIdx.x % hk;
  int si = 0;
  while (si + 1 < a.n_seqs && a.seqs[si + 1].row0 <= row) ++si;
  const int ns = a.seqs[si].n_splits;
  if (ns == 1) return;   // that sequence's queries were written by the split kernel itself
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int grp = tid >> 6, t = tid & 63;
  const float* base = a.partials + ((size_t)row * hk + head) * a.max_splits * rec;
  float M = kNegBig, L = 0.0f;
  floatx4 O = {0, 0, 0, 0};
#pragma unroll 2
  for (int sp = grp; sp < ns; sp += 16) {
    const float* pr = base + sp * rec;
    const float m = pr[h], l = pr[kPartialHeads + h];
    const floatx4 o = *(const floatx4*)(pr + 2 * kPartialHeads + h * D + 4 * t);
    const float mn = fmaxf(M, m);
    const float fa = __builtin_amdgcn_exp2f(M - mn), fb = __builtin_amdgcn_exp2f(m - mn);
    L = L * fa + l * fb;
#pragma unroll
    for (int k = 0; k < 4; ++k) O[k] = O[k] * fa + o[k] * fb;
    M = mn;
  }
  if (t == 0) {
    s_m[grp] = M;
    s_l[grp] = L;
  }
  s_o[grp][t] = O;
  __syncthreads();
  if (grp == 0) {
    float Mx = kNegBig;
#pragma unroll
    for (int k = 0; k < 16; ++k) Mx = fmaxf(Mx, s_m[k]);
    float Ls = 0.0f;
    floatx4 Os = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float f = __builtin_amdgcn_exp2f(s_m[k] - Mx);
      Ls += s_l[k] * f;
#pragma unroll
      for (int c = 0; c < 4; ++c) Os[c] += s_o[k][t][c] * f;
    }
    floatx4 r;
#pragma unroll
    for (int c = 0; c < 4; ++c) r[c] = Ls > 0.0f ? Os[c] / Ls : 0.0f;
    *(floatx4*)(a.out + ((size_t)row * a.n_q_heads + head * a.group + h) * D + 4 * t) = r;
  }
}

template <int NK, int NV, bool VAR>
hipError_t launch_mq_t(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(mq_kernel<NK, NV, VAR>, dim3(grid_x), dim3(512), s, e0, e1, a);
}

template <bool VAR>
hipError_t launch_mq_dispatch(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nk = a.g.k_bits, nv = a.g.v_bits;
#define KVQ_CASE(K, V) if (nk == K && nv == V) return launch_mq_t<K, V, VAR>(a, grid_x, s, e0, e1);
#define KVQ_ROW(K) KVQ_CASE(K, 2) KVQ_CASE(K, 3) KVQ_CASE(K, 4) KVQ_CASE(K, 5) KVQ_CASE(K, 6) KVQ_CASE(K, 7) KVQ_CASE(K, 8)
  KVQ_ROW(2) KVQ_ROW(3) KVQ_ROW(4) KVQ_ROW(5) KVQ_ROW(6) KVQ_ROW(7) KVQ_ROW(8)
#undef KVQ_ROW
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kvq
