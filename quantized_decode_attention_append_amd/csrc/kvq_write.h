// Device code of the cache writes (qN_0 or qN_1 quantization into the body, q8_0 into the 8-bit ring, the bf16 ring copy, the
// requantization of ring rows that leave the window), shared by the append kernels and by the decode kernel
// of a fused decode step. Quantization follows the symmetric qN_0 block format of the BeeLlama page (32
// values, one fp16 scale, no offset): d = amax / qmax in IEEE fp32, fp16 round-to-nearest-even saturating at
// 65504, codes rne(x / d16) clamped to [-qmax, qmax], stored biased by 2^(N-1). Every file that includes this
// is built with correctly rounded fp32 division, and every function below that does floating-point arithmetic
// turns contraction off for its own body (#pragma clang fp contract(off)), whatever the including file's
// -ffp-contract: no product is ever fused with an addition, so the codes are bit-identical to a plain IEEE
// evaluation in the kernels of the fused steps as well.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"

namespace kvq {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ inline float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
// IEEE binary16 bits of a bf16 value (round to nearest even; overflow to infinity): the f16 tail's stored form
__device__ inline uint16_t bf16_to_f16_bits(uint16_t b) {
  return __builtin_bit_cast(uint16_t, (_Float16)bf16_to_f32(b));
}

// ------------------------------------------------------------------------------ body write
//
// One work-group of 512 threads per (position tile, KV head); thread (kv, c) owns channel c of K (kv = 0)
// or V (kv = 1), so a block of 32 values is spread over 32 lanes (amax by lane shuffles) and even a single
// token is quantized with one division per thread. Codes are staged in LDS, then K rows and V tile words
// are packed from LDS.

__device__ inline float block_amax(float v) {
  // the 32 lanes of a block are lanes 0-31 or 32-63 of the wave
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Quantize one value of a block (all 32 lanes of the block call this together). Returns the biased code;
// *d16_bits receives the block's fp16 scale.
__device__ inline uint32_t quant_lane(float x, int n_bits, uint16_t* d16_bits) {
#pragma clang fp contract(off)
  const float amax = block_amax(fabsf(x));
  const float qmax = (float)((1 << (n_bits - 1)) - 1);
  float d = amax / qmax;                        // correctly rounded (see build flags)
  d = fminf(d, 65504.0f);
  const _Float16 h = (_Float16)d;               // RNE
  const float dh = (float)h;
  const int off = 1 << (n_bits - 1);
  if (dh == 0.0f) {
    *d16_bits = 0;
    return (uint32_t)off;
  }
  float c = rintf(x / dh);                      // round half to even
  c = fminf(fmaxf(c, -qmax), qmax);
  *d16_bits = __builtin_bit_cast(uint16_t, h);
  return (uint32_t)((int)c + off);
}

__device__ inline float block_min(float v) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float block_max(float v) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// qN_1 (a scale and a minimum per block; BeeLlama page, q2_1 .. q6_1 beside q5_1): d = (max - min) / (2^N - 1)
// in IEEE fp32, fp16 round-to-nearest-even saturating at 65504; the stored minimum is the block minimum rounded
// to fp16 (saturating at +/-65504); codes rne((x - m16) / d16) clamped to [0, 2^N - 1], zero when d16 is 0.
// All 32 lanes of the block call this together. Returns the code; *d16_bits, *m16_bits receive scale and minimum.
__device__ inline uint32_t quant_lane_min(float x, int n_bits, uint16_t* d16_bits, uint16_t* m16_bits) {
#pragma clang fp contract(off)
  const float mn = block_min(x);
  const float mx = block_max(x);
  const float levels = (float)((1 << n_bits) - 1);
  float d = (mx - mn) / levels;                 // correctly rounded (see build flags)
  d = fminf(d, 65504.0f);
  const _Float16 h = (_Float16)d;               // RNE
  const _Float16 mh = (_Float16)fminf(fmaxf(mn, -65504.0f), 65504.0f);
  *m16_bits = __builtin_bit_cast(uint16_t, mh);
  const float dh = (float)h;
  if (dh == 0.0f) {
    *d16_bits = 0;
    return 0u;
  }
  float c = rintf((x - (float)mh) / dh);        // round half to even
  c = fminf(fmaxf(c, 0.0f), levels);
  *d16_bits = __builtin_bit_cast(uint16_t, h);
  return (uint32_t)c;
}

// Token-axis K (a block is the 32 positions of one channel in a position tile): quantize the block held by one
// thread, xs[0..31], with the rules of quant_lane (symmetric qN_0) or quant_lane_min (qN_1). Writes the 32 codes
// (biased for qN_0) and the block's fp16 scale (and minimum).
__device__ inline void quant_block_local(const float* xs, int n_bits, bool with_min, uint8_t* u, uint16_t* d16_bits,
                                         uint16_t* m16_bits) {
#pragma clang fp contract(off)
  if (with_min) {
    float mn = xs[0], mx = xs[0];
    for (int t = 1; t < kTile; ++t) {
      mn = fminf(mn, xs[t]);
      mx = fmaxf(mx, xs[t]);
    }
    const float levels = (float)((1 << n_bits) - 1);
    float d = (mx - mn) / levels;
    d = fminf(d, 65504.0f);
    const _Float16 h = (_Float16)d;
    const _Float16 mh = (_Float16)fminf(fmaxf(mn, -65504.0f), 65504.0f);
    *m16_bits = __builtin_bit_cast(uint16_t, mh);
    const float dh = (float)h;
    *d16_bits = dh == 0.0f ? 0 : __builtin_bit_cast(uint16_t, h);
    for (int t = 0; t < kTile; ++t) {
      float c = dh == 0.0f ? 0.0f : rintf((xs[t] - (float)mh) / dh);
      u[t] = (uint8_t)fminf(fmaxf(c, 0.0f), levels);
    }
    return;
  }
  float amax = 0.0f;
  for (int t = 0; t < kTile; ++t) amax = fmaxf(amax, fabsf(xs[t]));
  const float qmax = (float)((1 << (n_bits - 1)) - 1);
  float d = amax / qmax;
  d = fminf(d, 65504.0f);
  const _Float16 h = (_Float16)d;
  const float dh = (float)h;
  const int off = 1 << (n_bits - 1);
  *d16_bits = dh == 0.0f ? 0 : __builtin_bit_cast(uint16_t, h);
  for (int t = 0; t < kTile; ++t) {
    float c = dh == 0.0f ? 0.0f : rintf(xs[t] / dh);
    c = fminf(fmaxf(c, -qmax), qmax);
    u[t] = (uint8_t)((int)c + off);
  }
}

// fp32 ring representation r(x) of one value: the bf16 value itself, its f16 rounding, or its q8_0 round trip.
__device__ inline float ring_rep(float x, int tail_dtype) {
#pragma clang fp contract(off)
  if (tail_dtype == 3) return (float)(_Float16)x;
  if (tail_dtype != 2) return x;
  uint16_t d;
  const uint32_t u = quant_lane(x, 8, &d);
  return (float)((int)u - 128) * f16_to_f32(d);   // exact product
}

// Value of channel c of position p (kv: 0 K, 1 V) read back from the ring, as fp32.
__device__ inline float ring_value(const Geometry& g, const uint8_t* slab, int kv, int head, int p, int c) {
#pragma clang fp contract(off)
  const int D = g.head_dim;
  const int NB = D / kBlock;
  const int NT = D / 16;
  const int R = g.ring_slots;
  const int slot = p % R;
  const int t = slot % kTile;
  const int lane = 16 * ((t % 16) / 4) + (c % 16);
  const int e = (t % 4) + 4 * (t / 16);
  const int b = c / kBlock;
  const int j = (c % kBlock) / 8;
  const int klane = 16 * j + (t % 16);   // K tile lane of (slot, channel)
  const size_t rt = (size_t)head * (R / kTile) + slot / kTile;   // ring tile (tile layout)
  if (g.tail_dtype == 1 || g.tail_dtype == 3) {   // 16-bit values: bf16 or f16
    const bool f16 = g.tail_dtype == 3;
    auto cv = [&](uint16_t bits) { return f16 ? f16_to_f32(bits) : bf16_to_f32(bits); };
    if (g.layout == 1) {   // position-major [slot][head][K row, V row]
      const int pair = g.ring_row_k + g.ring_row_v;
      const size_t off = kv ? rows_v_off(slot, head, g.n_kv_heads, pair, g.ring_row_k)
                            : rows_k_off(slot, head, g.n_kv_heads, pair);
      return cv(((const uint16_t*)(slab + g.k_ring + off))[c]);
    }
    if (kv == 0) {
      const uint16_t* kt = (const uint16_t*)(slab + g.k_ring + rt * g.ring_tile_k);
      return cv(kt[(((t / 16) * NB + b) * 64 + klane) * 8 + (c % 8)]);
    }
    const uint8_t* tile = slab + g.v_ring + rt * g.ring_tile_v;
    return cv(*((const uint16_t*)(tile + (size_t)(c / 16) * 64 * 16 + lane * 16) + e));
  }
  if (g.layout == 1) {
    const int pair = g.ring_row_k + g.ring_row_v;
    const uint8_t* row = slab + g.k_ring + (kv ? rows_v_off(slot, head, g.n_kv_heads, pair, g.ring_row_k)
                                               : rows_k_off(slot, head, g.n_kv_heads, pair));
    const float dh = f16_to_f32(((const uint16_t*)(row + NB * 32))[b]);
    return (float)((int)row[(j * NB + b) * 8 + (c % 8)] - 128) * dh;
  }
  if (kv == 0) {
    const uint8_t* kt = slab + g.k_ring + rt * g.ring_tile_k;
    const float dh = f16_to_f32(((const uint16_t*)(kt + 32 * D))[b * kTile + t]);
    return (float)((int)kt[512 * 8 * (t / 16) + lane_run_byte(klane, NB * 8 * 0 + 8 * b + (c % 8), NB * 8)] - 128) * dh;
  }
  const uint8_t* tile = slab + g.v_ring + rt * g.ring_tile_v;
  const float dh = f16_to_f32(((const uint16_t*)(tile + 32 * D))[b * kTile + t]);
  return (float)((int)tile[vtile_lane_byte(lane, (c / 16) * 8 + e, NT, 8)] - 128) * dh;
}

// OR one biased code u of (tile position t, channel c) into the body words that hold it. Body positions are
// written once after the slab was zeroed, so the target bits are zero and no read is needed; every word of
// a K tile / row belongs to one position, a V tile word is shared by up to 8 positions (hence the atomics).
// row: K (kv = 0) or V row of the position (row layout); tile: the position's K or V tile (tile layout).
__device__ inline void or_code(uint8_t* row, uint8_t* tile, bool rows, int kv, int n_bits, int t, int c, uint32_t u,
                               int D) {
  const int NB = D / kBlock, NT = D / 16;
  int row_off = 0, tile_off = 0;
  for (int p = 0; p < plane_count(n_bits); ++p) {
    const int w = plane_width(n_bits, p);
    const uint32_t field = (u >> plane_shift(n_bits, p)) & ((1u << w) - 1);
    int wbyte, bit, lane, e = 0;
    if (kv == 0 || rows) {
      const int b = c / kBlock, j = (c % kBlock) / 8, i = c % 8;
      if (w == 8) {
        wbyte = (8 * b + i) & ~3;
        bit = 8 * (i & 3);
      } else {
        wbyte = 4 * ((b * w) / 4);
        bit = 16 * (i & 1) + 4 * w * (b % (4 / w)) + w * (i >> 1);
      }
      lane = 16 * j + t % 16;
      uint8_t* dst = rows ? row + row_off + j * NB * w + wbyte
                          : tile + 512 * (n_bits * (t / 16)) + 16 * row_off + lane_run_byte(lane, wbyte, NB * w);
      if (field) atomicOr((uint32_t*)dst, field << bit);
    } else {
      const int n = c / 16;
      e = t % 4 + 4 * (t / 16);
      lane = 16 * ((t % 16) / 4) + c % 16;
      if (w == 8) {
        wbyte = (8 * n + e) & ~3;
        bit = 8 * (e & 3);
      } else {
        wbyte = 4 * ((n * w) / 4);
        bit = 16 * (e & 1) + 4 * w * (n % (4 / w)) + w * (e >> 1);
      }
      uint8_t* dst = tile + tile_off + vtile_lane_byte(lane, wbyte, NT, w);
      if (field) atomicOr((uint32_t*)dst, field << bit);
    }
    row_off += 4 * NB * w;
    tile_off += 64 * NT * w;
  }
}

// A work-group with at most this many positions ORs its codes straight into the body (no LDS staging).
constexpr int kDirectPositions = 4;

// LDS staging of one tile's codes: [K,V][tile position][channel].
typedef uint8_t WriteCodes[2][kTile][256];

// One work-group of 512 threads per (position tile, KV head): thread (kv, c) quantizes channel c of K (kv = 0)
// or V (kv = 1) for every position of the tile that the call writes. A: WriteArgs, or one role of StepArgs
// (the kernel argument itself, so that the item list is read in place). codes: the caller's LDS buffer.
// kMin = false compiles the qN_1 and token-axis K quantizers out (for callers that never write such bodies).
template <class A, bool kMin = true>
__device__ inline void body_write_wg(const A& a, int wg, int head, WriteCodes& codes) {
#pragma clang fp contract(off)
  const Geometry& g = a.g;
  int it = 0;
  while (it + 1 < a.n_items && a.items[it + 1].wg_begin <= wg) ++it;
  const WriteItem& w = a.items[it];
  const int tile = w.tile0 + (wg - w.wg_begin);
  const int D = g.head_dim;                    // 256: one channel per thread
  const int NB = D / kBlock;
  const int NT = D / 16;
  const int NK = a.dst_ring ? 8 : g.k_bits;
  const int NV = a.dst_ring ? 8 : g.v_bits;
  const int R = g.ring_slots;
  uint8_t* slab = g.arena + w.slab;

  const bool vrows = g.layout == 1;
  int row_k, row_v;
  size_t row_stride;   // row layout: bytes from one position's rows to the next one's (all heads' K and V rows)
  uint8_t* kbase;      // row layout: K row of position 0 of this head
  uint8_t* vbase;      // row layout: V row of position 0 of this head
  uint8_t* vtile;      // tile layout: this work-group's V tile
  uint8_t* ktile;      // tile layout: this work-group's K tile
  if (a.dst_ring) {
    row_k = row_v = g.ring_row_k;
    row_stride = (size_t)g.n_kv_heads * (row_k + row_v);
    kbase = slab + g.k_ring + rows_k_off(0, head, g.n_kv_heads, row_k + row_v);
    vbase = kbase + row_k;
    const size_t rt = (size_t)head * (R / kTile) + ((tile * kTile) % R) / kTile;
    ktile = slab + g.k_ring + rt * g.ring_tile_k;
    vtile = slab + g.v_ring + rt * g.ring_tile_v;
  } else {
    row_k = g.row_k;
    row_v = g.row_v;
    row_stride = (size_t)g.n_kv_heads * (row_k + row_v);
    kbase = slab + g.k_body + rows_k_off(0, head, g.n_kv_heads, row_k + row_v);
    vbase = kbase + row_k;
    ktile = slab + g.k_body + ((size_t)head * (g.cap32 / kTile) + tile) * g.tile_k;
    vtile = slab + g.v_body + ((size_t)head * (g.cap32 / kTile) + tile) * g.tile_v;
  }
  auto krow_of = [&](int p) { return kbase + (size_t)(a.dst_ring ? p % R : p) * row_stride; };
  auto vrow_of = [&](int p) { return vbase + (size_t)(a.dst_ring ? p % R : p) * row_stride; };
  const int t0 = max(w.p0 - tile * kTile, 0);
  const int t1 = min(w.p1 - tile * kTile, kTile);

  // ---- phase 1: codes of every (position, channel) of this call into LDS; scales straight to memory
  const int tid = threadIdx.x;
  const int kv = tid >> 8;
  const int c = tid & 255;
  const int b = c / kBlock;
  const int nb = kv ? NV : NK;
  const uint16_t* in = kv ? a.v_in : a.k_in;
  const float sig = (!a.dst_ring && g.kvarn)
                        ? f16_to_f32(((const uint16_t*)(slab + g.sigma))[((size_t)head * 2 + kv) * D + c])
                        : 1.0f;
  // few positions of the body (a decode step's evict): OR the codes in directly, no LDS round trip
  const bool direct = !a.dst_ring && t1 - t0 <= kDirectPositions;
  // the value of channel c at tile position t, as the body quantizes it
  auto value_at = [&](int t) {
    const int p = tile * kTile + t;
    float x;
    if (p >= w.len_old) {
      x = bf16_to_f32(in[((size_t)(w.src_row + p - w.len_old) * g.n_kv_heads + head) * D + c]);
      if (!a.dst_ring && R > 0) x = ring_rep(x, g.tail_dtype);   // through the ring representation
    } else {
      x = ring_value(g, slab, kv, head, p, c);
    }
    if (!a.dst_ring && g.kvarn) x = x / sig;
    return x;
  };
  if (kMin && kv == 0 && !a.dst_ring && g.k_axis) {
    // token-axis K: this thread's channel over the whole tile is one block (the host writes whole tiles here)
    float xs[kTile];
    for (int t = 0; t < kTile; ++t) xs[t] = value_at(t);
    uint8_t us[kTile];
    uint16_t dq, dm = 0;
    quant_block_local(xs, nb, g.k_min, us, &dq, &dm);
    for (int t = 0; t < kTile; ++t) codes[0][t][c] = us[t];
    ((uint16_t*)(ktile + 4 * D * NK))[c] = dq;                                          // scales [channel]
    if (g.k_min) ((uint16_t*)(ktile + 4 * D * NK + 2 * D))[c] = dm;                     // minima [channel]
  } else
  for (int t = t0; t < t1; ++t) {
    const int p = tile * kTile + t;
    const float x = value_at(t);
    uint16_t dq, dm = 0;
    const bool with_min = kMin && !a.dst_ring && (kv ? g.v_min : g.k_min);   // uniform over each 256-thread half
    const uint32_t u = with_min ? quant_lane_min(x, nb, &dq, &dm) : quant_lane(x, nb, &dq);
    if (direct) or_code(kv ? vrow_of(p) : krow_of(p), kv ? vtile : ktile, vrows, kv, nb, t, c, u, D);
    else codes[kv][t][c] = (uint8_t)u;
    if ((c % kBlock) == 0) {
      if (vrows) {
        uint16_t* sc = (uint16_t*)(kv ? vrow_of(p) + NB * 4 * NV : krow_of(p) + NB * 4 * NK);
        sc[b] = dq;
        if (with_min) sc[NB + b] = dm;                                               // minima after the scales
      } else if (kv == 0) {
        ((uint16_t*)(ktile + 4 * D * NK))[b * kTile + t] = dq;                       // [block][position]
        if (with_min) ((uint16_t*)(ktile + 4 * D * NK + 2 * NB * kTile))[t * NB + b] = dm;   // [position][block]
      } else {
        ((uint16_t*)(vtile + 4 * D * NV))[b * kTile + t] = dq;
        if (with_min) ((uint16_t*)(vtile + 4 * D * NV + 2 * NB * kTile))[b * kTile + t] = dm;
      }
    }
  }
  if (direct) return;   // uniform over the work-group
  __syncthreads();

  // ---- phase 2a: K rows (and, in the row layout, V rows) of the written positions, one 32-bit word per
  // work item
  for (int rkv = 0; rkv < (vrows ? 2 : 1); ++rkv) {
  const int NR = rkv ? NV : NK;
  const int words_per_row = NB * NR;           // sum over planes of 4 * NB * w / 4
  for (int item = tid; item < (t1 - t0) * words_per_row; item += 512) {
    const int t = t0 + item / words_per_row;
    int widx = item % words_per_row;
    int pl = 0, plane_off = 0;
    while (widx >= NB * plane_width(NR, pl)) {
      widx -= NB * plane_width(NR, pl);
      plane_off += 4 * NB * plane_width(NR, pl);
      ++pl;
    }
    const int wdt = plane_width(NR, pl);
    const int sh = plane_shift(NR, pl);
    const uint32_t m = (1u << wdt) - 1;
    const int wpj = NB * wdt / 4;               // words per lane group j in this plane
    const int j = widx / wpj;
    const int k = widx % wpj;
    uint32_t bits = 0;
    if (wdt == 8) {
      const int bb = k / 2, e0 = 4 * (k & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) bits |= (uint32_t)codes[rkv][t][32 * bb + 8 * j + e0 + e] << (8 * e);
    } else {
      const int per = 4 / wdt;
      for (int sl = 0; sl < per; ++sl) {
        const int bb = k * per + sl;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          bits |= ((uint32_t)(codes[rkv][t][32 * bb + 8 * j + e] >> sh) & m)
                  << (16 * (e & 1) + 4 * wdt * sl + wdt * (e >> 1));
      }
    }
    if (vrows) {
      uint8_t* row = rkv ? vrow_of(tile * kTile + t) : krow_of(tile * kTile + t);
      *(uint32_t*)(row + plane_off + 4 * widx) = bits;   // = j * NB * w + 4k
    } else {
      // K tile: subtile t / 16, lane 16 j + t % 16, byte 4k of the lane's run of this plane
      *(uint32_t*)(ktile + 512 * (NR * (t / 16)) + 16 * plane_off + lane_run_byte(16 * j + t % 16, 4 * k, NB * wdt)) =
          bits;
    }
  }
  }
  if (vrows) return;

  // ---- phase 2b: V tile words touched by this call (read-modify-write where partly covered)
  const int lane = tid & 63;
  const int q = tid >> 6;          // 0..7
  const int d16 = lane & 15;
  const int j = lane >> 4;
  uint32_t inmask = 0;   // bit e set when element e's tile position is written by this call
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tp = tile_pos(j, e);
    if (tp >= t0 && tp < t1) inmask |= 1u << e;
  }
  if (inmask == 0) return;
  // at most 3 planes x 4 words per thread (an 8-bit plane has 32 words per lane over 8 threads); the
  // fixed bounds keep every entry in registers
  constexpr int kSlots = 12;
  uint32_t* dst[kSlots];
  uint32_t bits[kSlots], mask[kSlots];
  bool use[kSlots];
  int vplane_off = 0;
#pragma unroll
  for (int pl = 0; pl < 3; ++pl) {
    const bool plane_ok = pl < plane_count(NV);
    const int wdt = plane_ok ? plane_width(NV, pl) : 1;
    const int sh = plane_ok ? plane_shift(NV, pl) : 0;
    const uint32_t m = (1u << wdt) - 1;
    const int run_dwords = NT * wdt / 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int slot = pl * 4 + kk;
      const int k = q + 8 * kk;
      use[slot] = plane_ok && k < run_dwords;
      uint32_t bt = 0, mk = 0;
      if (use[slot]) {
        if (wdt == 8) {
          const int n = k / 2;
          const int cc = 16 * n + d16;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int e = 4 * (k & 1) + bb;
            if (inmask & (1u << e)) {
              bt |= (uint32_t)codes[1][tile_pos(j, e)][cc] << (8 * bb);
              mk |= 0xFFu << (8 * bb);
            }
          }
        } else {
          const int per = 4 / wdt;
          for (int sl = 0; sl < per; ++sl) {
            const int n = k * per + sl;
            const int cc = 16 * n + d16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (inmask & (1u << e)) {
                const int pos = 16 * (e & 1) + 4 * wdt * sl + wdt * (e >> 1);
                bt |= ((uint32_t)(codes[1][tile_pos(j, e)][cc] >> sh) & m) << pos;
                mk |= m << pos;
              }
            }
          }
        }
      }
      dst[slot] = (uint32_t*)(vtile + vplane_off + vtile_lane_byte(lane, 4 * (use[slot] ? k : 0), NT, wdt));
      bits[slot] = bt;
      mask[slot] = mk;
    }
    if (plane_ok) vplane_off += 64 * NT * wdt;
  }
  if (!a.dst_ring) {
    // Body positions are written once after the slab was zeroed, so their bits in a shared word are still
    // zero: OR them in without reading the word first.
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
      if (use[k] && mask[k]) {
        if (mask[k] == 0xFFFFFFFFu) *dst[k] = bits[k];
        else atomicOr(dst[k], bits[k]);
      }
    return;
  }
  // ring slots are reused: read-modify-write
  uint32_t old[kSlots];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) old[k] = (use[k] && mask[k] != 0xFFFFFFFFu) ? *dst[k] : 0u;
#pragma unroll
  for (int k = 0; k < kSlots; ++k)
    if (use[k] && mask[k]) *dst[k] = (old[k] & ~mask[k]) | bits[k];
}

// ------------------------------------------------------------------------------ bf16 ring write

// One work-group of 512 threads per (position tile, KV head): thread (kv, c) copies channel c (bf16 tail) or
// rounds it to f16 (f16 tail).
template <class A>
__device__ inline void bf16_ring_write_wg(const A& a, int wg, int head) {
  const Geometry& g = a.g;
  int it = 0;
  while (it + 1 < a.n_items && a.items[it + 1].wg_begin <= wg) ++it;
  const WriteItem& w = a.items[it];
  const int tile = w.tile0 + (wg - w.wg_begin);
  const int D = g.head_dim;
  const int R = g.ring_slots;
  uint8_t* slab = g.arena + w.slab;
  const int kv = threadIdx.x >> 8;
  const int c = threadIdx.x & 255;
  const int t0 = max(w.p0 - tile * kTile, 0);
  const int t1 = min(w.p1 - tile * kTile, kTile);
  const uint16_t* in = kv ? a.v_in : a.k_in;
  for (int t = t0; t < t1; ++t) {
    const int p = tile * kTile + t;
    uint16_t v = in[((size_t)(w.src_row + p - w.len_old) * g.n_kv_heads + head) * D + c];
    if (g.tail_dtype == 3) v = bf16_to_f16_bits(v);   // f16 tail
    const int slot = p % R;
    if (g.layout == 1) {   // position-major [slot][head][K row, V row]
      const int pair = g.ring_row_k + g.ring_row_v;
      const size_t off = kv ? rows_v_off(slot, head, g.n_kv_heads, pair, g.ring_row_k)
                            : rows_k_off(slot, head, g.n_kv_heads, pair);
      ((uint16_t*)(slab + g.k_ring + off))[c] = v;
    } else if (kv == 0) {
      // [s][b][lane][8]: lane 16 j + slot % 16 holds channels 32b + 8j .. +7
      const int ts = slot % kTile;
      uint16_t* kt = (uint16_t*)(slab + g.k_ring + ((size_t)head * (R / kTile) + slot / kTile) * g.ring_tile_k);
      kt[(((ts / 16) * (D / kBlock) + c / kBlock) * 64 + 16 * ((c % kBlock) / 8) + ts % 16) * 8 + c % 8] = v;
    } else {
      uint8_t* vt = slab + g.v_ring + ((size_t)head * (R / kTile) + slot / kTile) * g.ring_tile_v;
      const int ts = slot % kTile;
      const int lane = 16 * ((ts % 16) / 4) + (c % 16);
      ((uint16_t*)(vt + (size_t)(c / 16) * 64 * 16 + lane * 16))[(ts % 4) + 4 * (ts / 16)] = v;
    }
  }
}

}  // namespace
}  // namespace kvq
