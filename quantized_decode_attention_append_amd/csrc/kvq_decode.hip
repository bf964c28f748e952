// Decode attention over the quantized cache: split-K flash decode with MFMA for the GQA group.
//
// Decode is bandwidth-bound: every step streams the whole cache of a full-attention layer (offload page, on
// the bytes a decode step reads), so the kernel is built around one pass over HBM per call:
//
// * grid (split, KV head, sequence); a work-group of 8 waves (two per SIMD) owns a set of 32-position tiles of
//   either the qN_0 body (every G-th tile, so that a KV head's work-groups stream one window of the body
//   together) or the tail ring (two KV paths per layer, Qwen3.8-27B page) and emits one partial (m, l, o) per
//   query head of the group;
// * each wave streams its tiles with 128-bit loads straight into registers: K rows are laid out so that
//   lane (row, j) reads the 8-code pieces of one position contiguously, V tiles so that lane (d16, j)
//   reads the MFMA B operand of P.V directly (no LDS transpose);
// * codes become exact fp16 integers with the "1024 + value" trick (AND-OR into the mantissa, one packed
//   FMA per pair and plane); QK = MFMA 16x16x32 per 32-value block (M = 16 positions, N = 8 heads of the
//   group as hi parts + 8 as lo parts of the exponent-shifted query), scaled per (position, block) in fp32;
// * online softmax in exp2 form with wave-wide max via DPP / shuffles;
// * P.V = MFMA with A = P * dv16 split into fp16 hi (rows 0-7) and lo (rows 8-15) parts, so the product
//   with the integer codes is accumulated to ~22 bits in fp32 (the hi/lo rows are summed at the end);
// * the bf16 tail uses bf16 MFMA directly on the stored values (hi/lo bf16 P).
// A second, fully parallel kernel merges the split partials (log-sum-exp).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"
#include "kvq_mfma.h"
#include "kvq_write.h"

// Waves per SIMD the decode kernel is compiled for: one 8-wave work-group per CU, up to 256 VGPRs a wave.
#ifndef KVQ_DECODE_WAVES_PER_EU
#define KVQ_DECODE_WAVES_PER_EU 2
#endif

namespace kvq {
namespace {


template <int W>
__device__ inline void load_words(const uint8_t* p, uint32_t* dst, int n_words) {
  // n_words is a compile-time multiple of 2 or 4 at every call site
  if (n_words % 4 == 0) {
    for (int k = 0; k < n_words; k += 4) {
      u32x4 v = ldnt(p + 4 * k);
      dst[k] = v[0]; dst[k + 1] = v[1]; dst[k + 2] = v[2]; dst[k + 3] = v[3];
    }
  } else {
    for (int k = 0; k < n_words; k += 2) {
      u32x2 v = __builtin_nontemporal_load((const u32x2*)(p + 4 * k));
      dst[k] = v[0]; dst[k + 1] = v[1];
    }
  }
}


// Raw bytes of one 32-position tile of a qN_0 store, as this lane loads them. The tile's fp16 scales
// (32 K rows x 16 bytes, 32 V positions x 16 bytes) are loaded one 16-byte chunk per lane and staged
// through LDS, because each lane needs the scales of 4 K rows and 8 V positions.
template <int NK, int NV>
struct TileRaw {
  static constexpr int NB = 8, NT = 16;
  static constexpr int w0k = Planes<NK>::w[0], w1k = Planes<NK>::w[1], w2k = Planes<NK>::w[2];
  static constexpr int w0v = Planes<NV>::w[0], w1v = Planes<NV>::w[1], w2v = Planes<NV>::w[2];
  static constexpr int nk0 = NB * w0k / 4, nk1 = w1k ? NB * w1k / 4 : 1, nk2 = w2k ? NB * w2k / 4 : 1;
  static constexpr int nv0 = NT * w0v / 4, nv1 = w1v ? NT * w1v / 4 : 1, nv2 = w2v ? NT * w2v / 4 : 1;
  uint32_t k0[2][nk0], k1[2][nk1], k2[2][nk2];   // K pieces of this lane's row in each 16-row subtile
  uint32_t v0[nv0], v1[nv1], v2[nv2];             // V pieces of this lane (16 n-tiles)
  u32x4 sc;                                       // 16 bytes of the K (lanes 0-31) or V (32-63) tile scales
};

// Tile loads go through buffer resources: the tile's base address and size sit in SGPRs and every lane's
// offset is fixed, so issuing the next tile's loads writes no VGPR besides their destinations (with VGPR
// addresses the compiler reused registers of loads still in flight and had to wait for them first). A
// resource of size 0 makes every load return zero without touching memory: the placeholder loads that keep
// the compiler's memory-counter waits exact when a wave has no next tile.
constexpr int kAuxNT = 2;                  // nontemporal (streaming) loads
constexpr int kOutOfRange = 0x7FFFFFF0;    // lane offset beyond any tile: the load returns zero

__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, bytes, 0x00020000);
}
__device__ inline u32x4 bld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAuxNT));
}
__device__ inline u32x2 bld8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kAuxNT));
}

// One plane run of a K subtile: lane l's run is [chunk][lane][min(16, 8w) B] from byte `off` of the tile.
template <int W>
__device__ inline void load_run(__amdgpu_buffer_rsrc_t r, int off, int lane, uint32_t* dst) {
  constexpr int words = 8 * W / 4;      // NB pieces of W bits x 8 codes
  if constexpr (words >= 4) {
#pragma unroll
    for (int c = 0; c < words / 4; ++c) {
      const u32x4 x = bld16(r, lane * 16, off + c * 1024);
      dst[4 * c] = x[0]; dst[4 * c + 1] = x[1]; dst[4 * c + 2] = x[2]; dst[4 * c + 3] = x[3];
    }
  } else {
    const u32x2 x = bld8(r, lane * 8, off);
    dst[0] = x[0]; dst[1] = x[1];
  }
}

// Issue the loads of one tile into `t` (kt / vt: the K and V tiles, kbytes / vbytes their sizes; live = false:
// placeholder loads that return zero). Every load reads 1 KiB (or 512 B) contiguous per wave. Scales first,
// then K, then V: the loads return in order, so staging the scales, QK and P.V each wait only for their own
// part of the tile.
template <int NK, int NV>
__device__ inline void load_tile_k(TileRaw<NK, NV>& t, const uint8_t* kt, int kbytes, const uint8_t* vt, int vbytes,
                                 bool live) {
  using T = TileRaw<NK, NV>;
  constexpr int NT = 16, D = 256;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt, live ? kbytes : 0);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt, live ? vbytes : 0);
  // scales, [block][position] fp16 in both tiles: lanes 0-31 take the K tile's 512 bytes, 32-63 the V tile's
  const int sck = lane < 32 ? 4 * D * NK + 16 * lane : kOutOfRange;
  const int scv = lane >= 32 ? 4 * D * NV + 16 * (lane - 32) : kOutOfRange;
  t.sc = bld16(rk, sck, 0);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int sub = 512 * NK * s;
    load_run<T::w0k>(rk, sub, lane, t.k0[s]);
    if constexpr (T::w1k > 0) load_run<T::w1k>(rk, sub + 512 * T::w0k, lane, t.k1[s]);
    if constexpr (T::w2k > 0) load_run<T::w2k>(rk, sub + 512 * (T::w0k + T::w1k), lane, t.k2[s]);
  }
}

template <int NK, int NV>
__device__ inline void load_tile_v(TileRaw<NK, NV>& t, const uint8_t* kt, int kbytes, const uint8_t* vt, int vbytes,
                                 bool live) {
  using T = TileRaw<NK, NV>;
  constexpr int NT = 16, D = 256;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt, live ? kbytes : 0);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt, live ? vbytes : 0);
  // scales, [block][position] fp16 in both tiles: lanes 0-31 take the K tile's 512 bytes, 32-63 the V tile's
  const int scv = lane >= 32 ? 4 * D * NV + 16 * (lane - 32) : kOutOfRange;
  t.sc |= bld16(rv, scv, 0);
#pragma unroll
  for (int c = 0; c < NT * T::w0v / 16; ++c) {
    const u32x4 x = bld16(rv, lane * 16, c * 1024);
    t.v0[4 * c] = x[0]; t.v0[4 * c + 1] = x[1]; t.v0[4 * c + 2] = x[2]; t.v0[4 * c + 3] = x[3];
  }
  if constexpr (T::w1v > 0) {
    const int p1 = 64 * NT * T::w0v;
#pragma unroll
    for (int c = 0; c < NT * T::w1v / 16; ++c) {
      const u32x4 x = bld16(rv, lane * 16, p1 + c * 1024);
      t.v1[4 * c] = x[0]; t.v1[4 * c + 1] = x[1]; t.v1[4 * c + 2] = x[2]; t.v1[4 * c + 3] = x[3];
    }
  }
  if constexpr (T::w2v > 0) {
    const u32x4 x = bld16(rv, lane * 16, 64 * NT * (T::w0v + T::w1v));
    t.v2[0] = x[0]; t.v2[1] = x[1]; t.v2[2] = x[2]; t.v2[3] = x[3];
  }
}

#define KVQ_SB __builtin_amdgcn_sched_barrier(0);

// LDS of the QK B operands: one [block][lane] array per K bit plane.
constexpr int kQbPlanes = 3;
constexpr int kQbHalf8 = kQbPlanes * 8 * 64;

// One 32-position tile of a qN_0 store (body, or the q8_0 ring). [lo, hi) are the valid positions.
// lane_mask is 0 on the hi-part lanes (rows 0-7 of the P operand) and ~0 on the lo-part lanes.
// s_sc: this wave's LDS copy of the tile's scales: K as [block][row], then V as [block][position].
template <int NK, int NV>
__device__ inline void qk_part(const TileRaw<NK, NV>& t, const u32x4* s_sc, const half8* qb,
                                    float qmul, int tile, int lo, int hi, float* x) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float sc[2][4];
  // K scales, transposed in LDS to [block][row]: the 4 rows 4g..4g+3 of a subtile are 8 contiguous bytes
  const uint16_t* s_dk = (const uint16_t*)s_sc;
  half8 kbias;   // -2^(N-1) * 2^(q_k - 24) per element: with the plane-0 query operand, minus the code bias
#pragma unroll
  for (int i = 0; i < 8; ++i)
    kbias[i] = (_Float16)(-ldexpf(1.0f, NK - 1 + dn_bitpos(Planes<NK>::w[0], 0, i) - 24));
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[s][r] = 0.0f;
  // Both 16-row subtiles block by block: one query operand read and one bias product serve both, and the two
  // subtiles' MFMA chains are independent, so each covers the other's latency. Block B's MFMAs are issued
  // before block B+1 is decoded, and their results consumed after that.
  KPlanes<NK> a0, a1;
  dn_piece<NK, 0>(t.k0[0], t.k1[0], t.k2[0], a0);
  dn_piece<NK, 0>(t.k0[1], t.k1[1], t.k2[1], a1);
#define KVQ_QK(B)                                                                                 \
  {                                                                                               \
    const half8 q0 = qb[B * 64 + lane];                                                           \
    floatx4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kbias, q0, floatx4{0, 0, 0, 0}, 0, 0, 0); \
    floatx4 c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kbias, q0, floatx4{0, 0, 0, 0}, 0, 0, 0); \
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.a[0], q0, c0, 0, 0, 0);                        \
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.a[0], q0, c1, 0, 0, 0);                        \
    if constexpr (Planes<NK>::n >= 2 && NK != 8) {                                                \
      const half8 q1 = qb[512 + B * 64 + lane];                                                   \
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.a[Planes<NK>::n >= 2 && NK != 8 ? 1 : 0], q1, c0, 0, 0, 0); \
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.a[Planes<NK>::n >= 2 && NK != 8 ? 1 : 0], q1, c1, 0, 0, 0); \
    }                                                                                             \
    if constexpr (Planes<NK>::n >= 3) {                                                           \
      const half8 q2 = qb[1024 + B * 64 + lane];                                                  \
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0.a[Planes<NK>::n >= 3 ? 2 : 0], q2, c0, 0, 0, 0); \
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1.a[Planes<NK>::n >= 3 ? 2 : 0], q2, c1, 0, 0, 0); \
    }                                                                                             \
    if constexpr (B < 7) {                                                                        \
      dn_piece<NK, (B < 7 ? B + 1 : 0)>(t.k0[0], t.k1[0], t.k2[0], a0);                           \
      dn_piece<NK, (B < 7 ? B + 1 : 0)>(t.k0[1], t.k1[1], t.k2[1], a1);                           \
    }                                                                                             \
    const u32x2 dk0 = *(const u32x2*)(s_dk + B * 32 + 4 * g);                                     \
    const u32x2 dk1 = *(const u32x2*)(s_dk + B * 32 + 16 + 4 * g);                                \
    sc[0][0] = fmaf(c0[0], lo_h(dk0[0]), sc[0][0]);                                               \
    sc[0][1] = fmaf(c0[1], hi_h(dk0[0]), sc[0][1]);                                               \
    sc[0][2] = fmaf(c0[2], lo_h(dk0[1]), sc[0][2]);                                               \
    sc[0][3] = fmaf(c0[3], hi_h(dk0[1]), sc[0][3]);                                               \
    sc[1][0] = fmaf(c1[0], lo_h(dk1[0]), sc[1][0]);                                               \
    sc[1][1] = fmaf(c1[1], hi_h(dk1[0]), sc[1][1]);                                               \
    sc[1][2] = fmaf(c1[2], lo_h(dk1[1]), sc[1][2]);                                               \
    sc[1][3] = fmaf(c1[3], hi_h(dk1[1]), sc[1][3]);                                               \
  }
  // one block at a time (sched barriers): bounds the live decoded operands
  KVQ_QK(0) KVQ_SB KVQ_QK(1) KVQ_SB KVQ_QK(2) KVQ_SB KVQ_QK(3) KVQ_SB
  KVQ_QK(4) KVQ_SB KVQ_QK(5) KVQ_SB KVQ_QK(6) KVQ_SB KVQ_QK(7) KVQ_SB
#undef KVQ_QK
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * s + r] = (sc[s][r] + dpp_ror8(sc[s][r])) * qmul;
  if (tile * kTile < lo || tile * kTile + kTile > hi) {   // a tile at either end of the range: mask positions
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = tile * kTile + 16 * s + 4 * g + r;
        if (pos < lo || pos >= hi) x[4 * s + r] = -INFINITY;
      }
  }
}

template <int NK, int NV>
__device__ inline void pv_part(WaveState& st, const TileRaw<NK, NV>& t, const u32x4* s_sc, const float* p, uint32_t lane_mask, uint32_t magic) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;

  // P masked to zero on the hi-part lanes: there the hi part below is P * dv itself
  float pm[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pm[i] = __uint_as_float(__float_as_uint(p[i]) & lane_mask);
  // V scales, transposed in LDS to [block][position]: this lane's positions T(g, 0..3) and T(g, 4..7)
  // are two runs of 4 fp16 values per block.
  const uint16_t* s_dv = (const uint16_t*)(s_sc + 32);
  // P.V: for block b, A = P * dv16 as fp16 hi (lane_mask = 0) or lo (lane_mask = ~0) parts
#define KVQ_PV(B)                                                                                   \
  {                                                                                                 \
    const u32x2 d0 = *(const u32x2*)(s_dv + B * 32 + 4 * g);                                         \
    const u32x2 d1 = *(const u32x2*)(s_dv + B * 32 + 16 + 4 * g);                                    \
    const uint32_t dw[4] = {d0[0], d0[1], d1[0], d1[1]};                                             \
    half8 a;                                                                                        \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                 \
      const half2v d = as_h2(dw[j]);                                                                \
      /* fma with +0 (not a product) so that it maps to a mixed-precision fma */                    \
      const _Float16 h0 = (_Float16)fmaf(pm[2 * j], (float)d[0], 0.0f);                             \
      const _Float16 h1 = (_Float16)fmaf(pm[2 * j + 1], (float)d[1], 0.0f);                         \
      a[2 * j] = (_Float16)fmaf(p[2 * j], (float)d[0], -(float)h0);                                 \
      a[2 * j + 1] = (_Float16)fmaf(p[2 * j + 1], (float)d[1], -(float)h1);                         \
    }                                                                                               \
    half8 b0 = decode_run_piece<NV, 2 * B>(t.v0, t.v1, t.v2, magic);                                \
    st.o[2 * B] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b0, st.o[2 * B], 0, 0, 0);              \
    half8 b1 = decode_run_piece<NV, 2 * B + 1>(t.v0, t.v1, t.v2, magic);                            \
    st.o[2 * B + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b1, st.o[2 * B + 1], 0, 0, 0);      \
  }
  KVQ_PV(0) KVQ_SB KVQ_PV(1) KVQ_SB KVQ_PV(2) KVQ_SB KVQ_PV(3) KVQ_SB
  KVQ_PV(4) KVQ_SB KVQ_PV(5) KVQ_SB KVQ_PV(6) KVQ_SB KVQ_PV(7) KVQ_SB
#undef KVQ_PV
}

// Next tile of the work-group's range for this wave: the waves of a work-group take tiles from a shared
// LDS counter, so a wave that gets fewer issue slots on its SIMD simply processes fewer tiles.
__device__ inline int grab_tile(int* s_next) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(s_next, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ inline const uint8_t* tile_ptr(const uint8_t* vbase, int tile_v, bool ring, int R, int t) {
  return vbase + (size_t)(ring ? ((t * kTile) % R) / kTile : t) * tile_v;
}

// Loop over tiles of a qN_0 store: this wave starts with tile t (already requested in `cur`) and then takes
// further tiles below tile_end from the work-group counter. During the compute of one tile the loads of
// the next are in flight. s_buf: this wave's two 1-KiB LDS buffers for tile scales.
template <int NK, int NV, bool UNROLL>
__device__ inline void run_quant_tiles(WaveState& st, TileRaw<NK, NV>& cur, TileRaw<NK, NV>& nxt, const half8* qb,
                                       float qmul, const uint8_t* kbase, int tile_k, bool ring, int R,
                                       const uint8_t* vbase, int tile_v, int tb, int ts, int t, int tile_end, int lo,
                                       int hi, uint32_t lane_mask, u32x4* s_buf, int* s_next) {
  const int lane = threadIdx.x & 63;
  if (t >= tile_end) return;
  uint32_t magic = kMagic;
  asm volatile("" : "+v"(magic));   // keep the fp16 magic in a VGPR (the mask takes the SGPR operand)
  // Stage one tile's scales into a wave-private LDS buffer (no work-group barrier needed).
  auto stage = [&](const TileRaw<NK, NV>& tr, u32x4* sb) {
    // the tiles hold their scales as [block][position]: K at sb[0..31], V at sb[32..63]
    sb[lane] = tr.sc;
  };
  if constexpr (UNROLL) {
    for (;;) {
      int nt = grab_tile(s_next);
      bool more = nt < tile_end;
      load_tile_k<NK, NV>(nxt, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts), tile_v,
                          more);
      stage(cur, s_buf);
      {
        float x[8], p[8];
        qk_part<NK, NV>(cur, s_buf, qb, qmul, tb + t * ts, lo, hi, x);
        load_tile_v<NK, NV>(nxt, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts),
                            tile_v, more);
        softmax_update(st, x, p);
        pv_part<NK, NV>(st, cur, s_buf, p, lane_mask, magic);
      }
      if (!more) break;
      t = nt;
      nt = grab_tile(s_next);
      more = nt < tile_end;
      load_tile_k<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts), tile_v,
                          more);
      stage(nxt, s_buf + 64);
      {
        float x[8], p[8];
        qk_part<NK, NV>(nxt, s_buf + 64, qb, qmul, tb + t * ts, lo, hi, x);
        load_tile_v<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts),
                            tile_v, more);
        softmax_update(st, x, p);
        pv_part<NK, NV>(st, nxt, s_buf + 64, p, lane_mask, magic);
      }
      if (!more) break;
      t = nt;
    }
    return;
  }
  int buf = 0;
  for (;;) {
    u32x4* sb = s_buf + 64 * buf;
    // the next tile's loads go out before this tile's scales are staged (which waits for this tile only)
    const int nt = grab_tile(s_next);
    const bool more = nt < tile_end;
    load_tile_k<NK, NV>(nxt, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts), tile_v,
                        more);
    stage(cur, sb);
    {
      float x[8], p[8];
      qk_part<NK, NV>(cur, sb, qb, qmul, tb + t * ts, lo, hi, x);
      load_tile_v<NK, NV>(nxt, tile_ptr(kbase, tile_k, ring, R, tb + (more ? nt : t) * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + (more ? nt : t) * ts),
                          tile_v, more);
      softmax_update(st, x, p);
      pv_part<NK, NV>(st, cur, sb, p, lane_mask, magic);
    }
    if (nt >= tile_end) break;
    t = nt;
    cur = nxt;
    buf ^= 1;
  }
}

// Whether the tile loop runs two tiles per trip (swapping the roles of the two register buffers instead of
// copying the prefetched one): only where both buffers and the decode temporaries fit in 256 VGPRs.
constexpr bool unroll_tiles(int nk, int nv) { return nk != 8 && nv <= 6 && nk + nv <= 11; }

// One 32-position tile of the bf16 tail ring (kt, vt: its K and V tiles). qb: the bf16 query B operands in
// LDS ([block][lane]).
__device__ inline void tile_bf16(WaveState& st, const bf16x8* qb, float qmul, const uint8_t* kt,
                                 const uint8_t* vt, int tile, int lo, int hi, bool lo_lane) {
  constexpr int D = 256, NT = 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float sc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // [s][b][lane][8 bf16]: lane (g, m16) holds channels 32b + 8g .. +7 of slot 16s + m16
    bf16x8 kk[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) kk[b] = __builtin_nontemporal_load((const bf16x8*)(kt + ((s * 8 + b) * 64 + lane) * 16));
    floatx4 c = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[b], qb[b * 64 + lane], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[s][r] = c[r];
  }
  float x[8], p[8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = tile * kTile + 16 * s + 4 * g + r;
      x[4 * s + r] = (pos >= lo && pos < hi) ? sc[s][r] * qmul : -INFINITY;
    }
  softmax_update(st, x, p);
  bf16x8 a;
  const float kf = lo_lane ? 1.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)p[i];
    a[i] = (__bf16)fmaf(-kf, (float)h, p[i]);
  }
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += 4) {
    bf16x8 vv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vv[k] = __builtin_nontemporal_load((const bf16x8*)(vt + (n0 + k) * 1024 + lane * 16));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      st.o[n0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vv[k], st.o[n0 + k], 0, 0, 0);
  }
}

// One 32-position tile of the f16 tail ring: as tile_bf16 with fp16 MFMA. The query B operand holds fp16 hi
// parts in columns 0-7 and lo parts in columns 8-15 (the bf16 query is not always exact in fp16), so a score
// is the sum of columns h and h + 8 (one DPP rotation by 8 within the 16-lane row).
__device__ inline void tile_f16(WaveState& st, const half8* qb, float qmul, const uint8_t* kt,
                                const uint8_t* vt, int tile, int lo, int hi, bool lo_lane) {
  constexpr int NT = 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float sc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    half8 kk[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) kk[b] = __builtin_nontemporal_load((const half8*)(kt + ((s * 8 + b) * 64 + lane) * 16));
    floatx4 c = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk[b], qb[b * 64 + lane], c, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[s][r] = c[r] + dpp_ror8(c[r]);   // hi column + lo column
  }
  float x[8], p[8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = tile * kTile + 16 * s + 4 * g + r;
      x[4 * s + r] = (pos >= lo && pos < hi) ? sc[s][r] * qmul : -INFINITY;
    }
  softmax_update(st, x, p);
  half8 a;
  const float kf = lo_lane ? 1.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)p[i];
    a[i] = (_Float16)fmaf(-kf, (float)h, p[i]);
  }
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += 4) {
    half8 vv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vv[k] = __builtin_nontemporal_load((const half8*)(vt + (n0 + k) * 1024 + lane * 16));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      st.o[n0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, vv[k], st.o[n0 + k], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ the split kernel

struct QArgs {
  const uint16_t* qgroup; // the query heads of this KV head's group (bf16 [group][D]), a uniform address
  int group;
  const uint16_t* sig;    // KVarN sigma of this KV head ([K,V][D] fp16)
  bool use_sigma, head_ok, lo_lane;
  float scale;
};

// A qN_0 store path (body, or q8_0 ring): issue the first tile's loads, build the exponent-shifted query
// operands (times KVarN sigma) in LDS, then run the tile loop. All waves of the work-group call this.
template <int NK, int NV, bool EARLY>
__device__ inline void quant_path(WaveState& st, const QArgs& qa, half8* s_qb, const uint8_t* kbase, int tile_k,
                                  bool ring, int R, const uint8_t* vbase, int tile_v, int tb, int ts, int wb, int we,
                                  int lo, int hi, uint32_t lane_mask, u32x4* sbuf, int* s_next, float* s_amax) {
  constexpr int NB = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: tile addresses stay scalar
  const int gq = lane >> 4;
  TileRaw<NK, NV> cur, nxt;
  // Wave w prepares block w of the query operand. Its query (and KVarN sigma) loads go out before the
  // first tile's: issued behind the tile loads they would wait for the work-group's tile traffic.
  // this lane's head row, computed here from the lane id (a per-lane pointer kept from the kernel's start
  // would stay live through the other wave path's tile loop)
  const int hh = lane & 7;
  const u32x4 qraw = *(const u32x4*)(qa.qgroup + (hh < qa.group ? hh : 0) * 256 + 32 * wave + 8 * gq);
  u32x4 sraw = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};   // fp16 1.0
  if (qa.use_sigma) sraw = *(const u32x4*)(qa.sig + 32 * wave + 8 * gq);
  KVQ_SB
  const int t0 = wb < we ? wb : we - 1;
  if constexpr (EARLY) {
    load_tile_k<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + t0 * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + t0 * ts), tile_v, wb < we);
    load_tile_v<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + t0 * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + t0 * ts), tile_v, wb < we);
  }
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {   // q times sigma is exact in fp32 (8 + 11 bits)
    x[2 * k] = __uint_as_float(qraw[k] << 16) * lo_h(sraw[k]);
    x[2 * k + 1] = __uint_as_float(qraw[k] & 0xFFFF0000u) * hi_h(sraw[k]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max_16_32(amax);
  if (lane < 16) s_amax[wave * 16 + lane] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 8; ++w) amax = fmaxf(amax, s_amax[w * 16 + (lane & 15)]);
  // exponent-shifted query of this lane's head (|q| < 2^9, so that the plane weights of up to 2^6 stay in
  // fp16 range), split into fp16 hi (cols 0-7) and lo (cols 8-15); one weighted copy per K bit plane
  const int e = amax > 0.0f ? ilogbf(amax) - 8 : 0;
  {
    float part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xs = ldexpf(x[i], -e);
      const _Float16 h = (_Float16)xs;
      const _Float16 l = (_Float16)(xs - (float)h);
      part[i] = qa.head_ok ? (float)(qa.lo_lane ? l : h) : 0.0f;
    }
#pragma unroll
    for (int p = 0; p < Planes<NK>::n; ++p) {
      half8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = Planes<NK>::w[p];
        const int slot = w == 8 ? 0 : wave % (4 / w);
        v[i] = (_Float16)ldexpf(part[i], Planes<NK>::sh[p] - dn_bitpos(w, slot, i));   // exact: power of two
      }
      s_qb[p * 512 + wave * 64 + lane] = v;
    }
  }
  __syncthreads();
  if constexpr (!EARLY) {
    load_tile_k<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + t0 * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + t0 * ts), tile_v, wb < we);
    load_tile_v<NK, NV>(cur, tile_ptr(kbase, tile_k, ring, R, tb + t0 * ts), tile_k, tile_ptr(vbase, tile_v, ring, R, tb + t0 * ts), tile_v, wb < we);
  }
  const float qmul = qa.scale * kLog2e * ldexpf(1.0f, e + 24);
  run_quant_tiles<NK, NV, unroll_tiles(NK, NV)>(st, cur, nxt, s_qb, qmul, kbase, tile_k, ring, R, vbase, tile_v, tb, ts, wb, we, lo, hi, lane_mask,
                          sbuf, s_next);
}

// One write of a fused decode step, with the members the shared write code reads.
struct StepWriteView {
  const Geometry& g;
  const uint16_t* k_in;
  const uint16_t* v_in;
  int dst_ring;
  int n_items;
  WriteItem items[1];
};

// The writes of a fused decode step that fall to this work-group, done by all its threads before any of them
// reads the cache: the last ring split writes the appended token into the ring, the last body split
// requantizes the ring rows leaving the window into the body (the tiles they land in belong to that split).
__device__ inline void step_writes(const DecodeArgs& a, const DecodeSeq& S, int si, int head, int split, bool is_ring,
                                   WriteCodes& codes) {
  const int n_splits = S.n_body_splits + S.n_ring_splits;
  if (is_ring && split == n_splits - 1 && S.app_pos >= 0) {
    const StepWriteView w{a.g, a.k_in, a.v_in, 1, 1,
                          {WriteItem{S.slab, S.app_pos, S.app_pos + 1, S.app_pos, si, S.app_pos / kTile, 0}}};
    if (a.g.tail_dtype != 2) bf16_ring_write_wg(w, 0, head);   // bf16 or f16 values
    else body_write_wg<StepWriteView, false>(w, 0, head, codes);
  } else if (!is_ring && split == S.n_body_splits - 1 && S.ev1 > S.ev0) {
    // (a cache with a qN_1 body never runs the fused step: the host plans it as separate calls)
    const StepWriteView w{a.g, a.k_in, a.v_in, 0, 1,
                          {WriteItem{S.slab, S.ev0, S.ev1, S.len, 0, S.ev0 / kTile, 0}}};
    body_write_wg<StepWriteView, false>(w, 0, head, codes);
  } else {
    return;
  }
  // the writes are complete (and visible to this work-group) before its waves load any tile
  __threadfence_block();
  __syncthreads();
}

// One work-group of 8 waves (two per SIMD) per split; the host sizes the splits so that there is about one
// work-group per CU. The waves claim the split's tiles one at a time from an LDS counter (the two waves of
// a SIMD do not get equal issue slots, so a static share would leave one of them finishing late); the
// waves' partial results are merged in LDS into one partial record.
template <int NK, int NV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(KVQ_DECODE_WAVES_PER_EU, KVQ_DECODE_WAVES_PER_EU)))
void decode_kernel(DecodeArgs a) {
  constexpr int D = 256, NB = 8, NT = 16, NW = 8;
  // One 64 KiB LDS region serves three phases in turn, each ended by a work-group barrier: the codes of a fused
  // step's writes; then the QK B operands (24 KiB) and the waves' tile scales (16 KiB); then the waves' partial
  // outputs (64 KiB). Two work-groups fit one CU.
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kPartialHeads * NW * D * 4];
  static_assert(sizeof(WriteCodes) <= sizeof(s_lds), "codes");
  static_assert(kQbHalf8 * sizeof(half8) + NW * 2 * 64 * sizeof(u32x4) <= sizeof(s_lds), "operands and scales");
  float (*s_o)[kPartialHeads][D] = (float (*)[kPartialHeads][D])s_lds;
  half8* s_qb = (half8*)s_lds;                                                     // QK B operands
  u32x4 (*s_scales)[2][64] = (u32x4 (*)[2][64])(s_lds + kQbHalf8 * sizeof(half8));   // per wave, double-buffered
  __shared__ float s_ml[NW][2][kPartialHeads];
  __shared__ int s_next;                   // next unclaimed tile of this split
  __shared__ float s_amax[8 * 16];         // per wave: |q| maximum of each head over the wave's block

  // flattened grid: (sequence, KV head, split)
  const Geometry& g = a.g;
  int rem = blockIdx.x;
  int si = 0;
  for (;;) {
    const int n = g.n_kv_heads * (a.seqs[si].n_body_splits + a.seqs[si].n_ring_splits);
    if (rem < n || si + 1 >= a.n_seqs) break;
    rem -= n;
    ++si;
  }
  const DecodeSeq S = a.seqs[si];
  const int n_splits = S.n_body_splits + S.n_ring_splits;
  const int head = rem / n_splits;
  const int split = rem % n_splits;
  const bool is_ring = split >= S.n_body_splits;
  if (a.step) step_writes(a, S, si, head, split, is_ring, *(WriteCodes*)s_lds);
  const int tail = g.tail_dtype;
  const int R = g.ring_slots;
  const uint8_t* slab = g.arena + S.slab;

  int seg_begin, seg_tiles, nsp, sp, lo, hi;
  if (!is_ring) {
    seg_begin = 0;
    seg_tiles = (S.body_len + kTile - 1) / kTile;
    nsp = S.n_body_splits;
    sp = split;
    lo = 0;
    hi = S.body_len;
  } else {
    seg_begin = S.ring_tile0;
    seg_tiles = (S.len + kTile - 1) / kTile - S.ring_tile0;
    nsp = S.n_ring_splits;
    sp = split - S.n_body_splits;
    lo = S.body_len;
    hi = S.len;
  }
  // this split's tiles are tb + k * ts for k in [0, n_tiles): wave w starts with k = w, further k come from
  // s_next. Body splits interleave: split sp < nsp - 1 takes every (nsp - 1)-th tile of [0, L) from tile sp on,
  // so that at any time the work-groups of a KV head stream one window of the body together, and the last split
  // takes the contiguous tiles [L, seg_tiles) at the end, which hold the rows a fused decode step requantizes
  // (that split writes them before it reads anything; last_tb > 0 gives it fewer tiles for the time it spends
  // writing). The ring segment is split into contiguous ranges; its last split holds the appended position.
  int tb, te, ts = 1;
  if (!is_ring && nsp > 1) {
    const int L = S.last_tb > 0 ? S.last_tb : seg_tiles - (seg_tiles / nsp > 1 ? seg_tiles / nsp : 1);
    if (sp == nsp - 1) {
      tb = L;
      te = seg_tiles;
    } else {
      tb = sp;
      te = L;
      ts = nsp - 1;
    }
  } else {
    tb = seg_begin + (int)((long)sp * seg_tiles / nsp);
    te = seg_begin + (int)((long)(sp + 1) * seg_tiles / nsp);
  }
  const int n_tiles = te > tb ? (te - tb + ts - 1) / ts : 0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile addresses stay scalar
  const int lane = tid & 63;
  const int wb = wave;
  const int we = n_tiles;
  if (tid == 0) s_next = NW;   // published by the work-group barrier before the first tile loop

  const int m16 = lane & 15;
  const int gq = lane >> 4;
  const int hh = m16 & 7;
  const bool lo_lane = m16 >= 8;
  const bool head_ok = hh < a.group;
  const int qh = head * a.group + hh;
  const uint16_t* qrow = a.q + ((size_t)si * a.n_q_heads + (head_ok ? qh : 0)) * D;
  const bool use_sigma = g.kvarn && !is_ring;
  const uint16_t* sig = (const uint16_t*)(slab + g.sigma) + (size_t)head * 2 * D;

  WaveState st;
  st.m = kNegBig;
  st.l = 0.0f;
#pragma unroll
  for (int n = 0; n < NT; ++n) st.o[n] = floatx4{0, 0, 0, 0};

  // channels of this lane's B operand: 32b + 8*gq + i
  if (is_ring && (tail == 1 || tail == 3)) {
    // B operands of QK: bf16 ring: the bf16 query, columns 8-15 repeating heads 0-7 so the lo-part lanes see
    // the same scores; f16 ring: fp16 hi parts in columns 0-7, lo parts in columns 8-15
    u32x4* qb = (u32x4*)s_qb;
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u32x4 w = *(const u32x4*)(qrow + 32 * b + 8 * gq);
        if (tail == 3) {
          half8 v;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float q = __uint_as_float((w[i >> 1] >> (16 * (i & 1))) << 16);
            const _Float16 h = (_Float16)q;
            v[i] = lo_lane ? (_Float16)(q - (float)h) : h;
          }
          w = __builtin_bit_cast(u32x4, v);
        }
        if (!head_ok) w = u32x4{0u, 0u, 0u, 0u};
        qb[b * 64 + lane] = w;
      }
    }
    __syncthreads();
    const float qmul = a.scale * kLog2e;
    for (int k = wb; k < we; k = grab_tile(&s_next)) {
      const int t = tb + k * ts;
      const size_t rt = (size_t)head * (R / kTile) + ((t * kTile) % R) / kTile;
      const uint8_t* kt = slab + g.k_ring + rt * g.ring_tile_k;
      const uint8_t* vt = slab + g.v_ring + rt * g.ring_tile_v;
      if (tail == 3) tile_f16(st, (const half8*)qb, qmul, kt, vt, t, lo, hi, lo_lane);
      else tile_bf16(st, (const bf16x8*)qb, qmul, kt, vt, t, lo, hi, lo_lane);
    }
  } else {
    const uint32_t lane_mask = lo_lane ? 0xFFFFFFFFu : 0u;
    const QArgs qa{a.q + ((size_t)si * a.n_q_heads + (size_t)head * a.group) * D, a.group, sig, use_sigma, head_ok,
                   lo_lane, a.scale};
    u32x4* sbuf = &s_scales[wave][0][0];
    if (!is_ring) {
      const uint8_t* kbase = slab + g.k_body + (size_t)head * (g.cap32 / kTile) * g.tile_k;
      const uint8_t* vbase = slab + g.v_body + (size_t)head * (g.cap32 / kTile) * g.tile_v;
      // waves 0-3 (one per SIMD) request their first tile at once, waves 4-7 only once the query is set
      // up: a smaller first burst reaches every SIMD sooner
      if (wave < 4)
        quant_path<NK, NV, true>(st, qa, s_qb, kbase, g.tile_k, false, 1, vbase, g.tile_v, tb, ts, wb, we, lo, hi, lane_mask,
                                 sbuf, &s_next, s_amax);
      else {
        // the later-starting wave of each SIMD gets issue priority, so that both finish together
        __builtin_amdgcn_s_setprio(1);
        quant_path<NK, NV, false>(st, qa, s_qb, kbase, g.tile_k, false, 1, vbase, g.tile_v, tb, ts, wb, we, lo, hi, lane_mask,
                                  sbuf, &s_next, s_amax);
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      const uint8_t* kbase = slab + g.k_ring + (size_t)head * (R / kTile) * g.ring_tile_k;
      const uint8_t* vbase = slab + g.v_ring + (size_t)head * (R / kTile) * g.ring_tile_v;
      quant_path<8, 8, true>(st, qa, s_qb, kbase, g.ring_tile_k, true, R, vbase, g.ring_tile_v, tb, ts, wb, we, lo, hi,
                             lane_mask, sbuf, &s_next, s_amax);
    }
  }

  // ---- wave epilogue: l over the lanes of a head; o = hi rows + lo rows
  const float lsum = sum_xor32(sum_xor16(lo_lane ? 0.0f : st.l));
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[n][r] = sum_xor32(st.o[n][r]);
  if (lane < 8) {
    s_ml[wave][0][lane] = st.m;
    s_ml[wave][1][lane] = lsum;
  }
  __syncthreads();
  // this wave's factor 2^(m_w - M) for the heads of its accumulator rows (4 gq + r), M = max over the waves
  if (gq < 2) {
    float f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * gq + r;
      float M = kNegBig;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0][h]);
      f[r] = __builtin_amdgcn_exp2f(s_ml[wave][0][h] - M);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][4 * gq + r][16 * n + m16] = st.o[n][r] * f[r];
  }
  __syncthreads();

  // ---- sum the waves' scaled outputs and write the partial of this split (512 threads: 2 heads x 256 channels)
  float* part = a.partials + (((size_t)si * g.n_kv_heads + head) * a.max_splits + split) * (kPartialHeads * (D + 2));
  const int c = tid & 255;
  const float vs = use_sigma ? h2f(sig[D + c]) : 1.0f;
#pragma unroll
  for (int h = tid >> 8; h < kPartialHeads; h += 2) {
    float O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) O += s_o[w][h][c];
    part[2 * kPartialHeads + h * D + c] = O * vs;
  }
  if (tid < kPartialHeads) {
    float M = kNegBig, L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0][tid]);
#pragma unroll
    for (int w = 0; w < NW; ++w) L += s_ml[w][1][tid] * __builtin_amdgcn_exp2f(s_ml[w][0][tid] - M);
    part[tid] = M;
    part[kPartialHeads + tid] = L;
  }
}

// ------------------------------------------------------------------ merge of the split partials

// One work-group per (sequence, KV head, query head, 16-channel chunk): 16 groups of 16 threads each fold a
// strided share of the splits into a running (max, sum, output) in one pass (online log-sum-exp, exp2
// domain), then the 16 groups are merged: out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int D = 256;
  constexpr size_t rec = kPartialHeads * (D + 2);
  __shared__ float s_m[16], s_l[16], s_o[16][17];
  const int si = blockIdx.x / a.n_kv_heads;
  const int head = blockIdx.x % a.n_kv_heads;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int c = blockIdx.z * 16 + (tid & 15);
  const int grp = tid >> 4;
  const int ns = a.n_splits[si];
  const float* base = a.partials + ((size_t)si * a.n_kv_heads + head) * a.max_splits * rec;
  float M = kNegBig, L = 0.0f, O = 0.0f;
#pragma unroll 4
  for (int sp = grp; sp < ns; sp += 16) {
    const float* pr = base + sp * rec;
    const float m = pr[h], l = pr[kPartialHeads + h], o = pr[2 * kPartialHeads + h * D + c];
    const float mn = fmaxf(M, m);
    const float fa = __builtin_amdgcn_exp2f(M - mn), fb = __builtin_amdgcn_exp2f(m - mn);
    L = L * fa + l * fb;
    O = O * fa + o * fb;
    M = mn;
  }
  if ((tid & 15) == 0) {
    s_m[grp] = M;
    s_l[grp] = L;
  }
  s_o[grp][tid & 15] = O;
  __syncthreads();
  if (tid < 16) {
    float Mx = kNegBig;
#pragma unroll
    for (int k = 0; k < 16; ++k) Mx = fmaxf(Mx, s_m[k]);
    float Ls = 0.0f, Os = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float f = __builtin_amdgcn_exp2f(s_m[k] - Mx);
      Ls += s_l[k] * f;
      Os += s_o[k][tid] * f;
    }
    a.out[((size_t)si * a.n_q_heads + head * a.group + h) * D + blockIdx.z * 16 + tid] = Ls > 0.0f ? Os / Ls : 0.0f;
  }
}

template <int NK, int NV>
hipError_t launch_decode_t(const DecodeArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(decode_kernel<NK, NV>, dim3(grid_x), dim3(512), s, e0, e1, a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nk = a.g.k_bits, nv = a.g.v_bits;
#define KVQ_CASE(K, V) if (nk == K && nv == V) return launch_decode_t<K, V>(a, grid_x, s, e0, e1);
#define KVQ_ROW(K) KVQ_CASE(K, 2) KVQ_CASE(K, 3) KVQ_CASE(K, 4) KVQ_CASE(K, 5) KVQ_CASE(K, 6) KVQ_CASE(K, 7) KVQ_CASE(K, 8)
  KVQ_ROW(2) KVQ_ROW(3) KVQ_ROW(4) KVQ_ROW(5) KVQ_ROW(6) KVQ_ROW(7) KVQ_ROW(8)
#undef KVQ_ROW
#undef KVQ_CASE
  return hipErrorInvalidValue;
}


hipError_t launch_combine(const CombineArgs& a, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(combine_kernel, dim3(a.n_seqs * a.n_kv_heads, a.group, a.head_dim / 16), dim3(256), s, e0, e1, a);
}


}  // namespace kvq
