// Decode attention over the quantized cache: split-K flash decode with MFMA for the GQA group.
//
// Decode is bandwidth-bound: every step streams the whole cache of a full-attention layer (offload page,
// "decode is a bandwidth problem"), so the kernel is built around one pass over HBM per call:
//
// * grid (split, KV head, sequence); a work-group of 4 waves owns a contiguous range of 32-position tiles
//   of either the qN_0 body or the tail ring (two KV paths per layer, Qwen3.8-27B page) and emits one
//   partial (m, l, o) per query head of the group;
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
// A second small kernel merges the partials (log-sum-exp).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kMagic = 0x64006400u;   // fp16 1024.0 in both halves

__device__ inline half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ inline uint32_t as_u(half2v x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ------------------------------------------------------------------ code planes (compile time)

template <int N> struct Planes;
template <> struct Planes<2> { static constexpr int n = 1; static constexpr int w[3] = {2, 0, 0}; static constexpr int sh[3] = {0, 0, 0}; };
template <> struct Planes<3> { static constexpr int n = 2; static constexpr int w[3] = {2, 1, 0}; static constexpr int sh[3] = {0, 2, 0}; };
template <> struct Planes<4> { static constexpr int n = 1; static constexpr int w[3] = {4, 0, 0}; static constexpr int sh[3] = {0, 0, 0}; };
template <> struct Planes<5> { static constexpr int n = 2; static constexpr int w[3] = {4, 1, 0}; static constexpr int sh[3] = {0, 4, 0}; };
template <> struct Planes<6> { static constexpr int n = 2; static constexpr int w[3] = {4, 2, 0}; static constexpr int sh[3] = {0, 4, 0}; };
template <> struct Planes<7> { static constexpr int n = 3; static constexpr int w[3] = {4, 2, 1}; static constexpr int sh[3] = {0, 4, 6}; };
template <> struct Planes<8> { static constexpr int n = 1; static constexpr int w[3] = {8, 0, 0}; static constexpr int sh[3] = {0, 0, 0}; };

template <int N>
constexpr int plane_bytes_per_piece_sum() {
  int s = 0;
  for (int p = 0; p < Planes<N>::n; ++p) s += Planes<N>::w[p];
  return s;   // == N
}

// Bit offset (within a 16-bit half) of pair k of piece slot `slot` in a plane of width w.
constexpr int pair_offset(int w, int slot, int k) { return 4 * w * slot + w * k; }
// Right shift applied before extraction so that the field sits in mantissa bits [0, 10).
constexpr int pair_pre_shift(int w, int slot, int k) { return (pair_offset(w, slot, k) + w > 10) ? 8 : 0; }

// Pair k (elements 2k, 2k+1) of a w<8 piece held in `word` at slot `slot`: two fp16 magic values
// 1024 + 2^q * v. Returns the packed halves and the scale exponent q.
template <int W, int SLOT, int K>
__device__ inline uint32_t extract_pair(uint32_t word) {
  constexpr int q = pair_offset(W, SLOT, K) - pair_pre_shift(W, SLOT, K);
  constexpr uint32_t m = ((1u << W) - 1) << q;
  constexpr uint32_t mask = m | (m << 16);
  constexpr int s = pair_pre_shift(W, SLOT, K);
  return ((word >> s) & mask) | kMagic;
}
template <int W, int SLOT, int K>
constexpr int pair_q() { return pair_offset(W, SLOT, K) - pair_pre_shift(W, SLOT, K); }

// Piece view: for each plane, the word holding the piece and its slot.
struct PieceWords {
  uint32_t w[3];     // word of plane p (for w = 8: w[0] low dword, w[1] high dword)
};

// Decode one piece (8 codes) into exact fp16 signed values c = u - 2^(N-1). SLOTS are the piece's slot
// index in each plane's word (0 for w >= 4).
template <int N, int S1, int S2>
__device__ inline half8 decode_piece(const PieceWords& pw) {
  constexpr int off = 1 << (N - 1);
  u32x4 r;
  if constexpr (N == 8) {
    // bytes e0..e7 -> (0x64, e) halves via byte permute
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t src = pw.w[k >> 1];
      const uint32_t sel = (k & 1) ? 0x04030402u : 0x04010400u;
      const uint32_t hv = __builtin_amdgcn_perm(0x64646464u, src, sel);
      r[k] = as_u(as_h2(hv) - as_h2(0x64006400u + (uint32_t)(off | (off << 16))));   // exact: 1024+u - (1024+off)
    }
    return __builtin_bit_cast(half8, r);
  } else {
    constexpr int np = Planes<N>::n;
    constexpr int w0 = Planes<N>::w[0];
    constexpr int w1 = Planes<N>::w[1];
    constexpr int w2 = Planes<N>::w[2];
    constexpr int sh1 = Planes<N>::sh[1];
    constexpr int sh2 = Planes<N>::sh[2];
    // plane 0 always sits at slot 0 for w0 = 4; for w0 = 2 (N = 2, 3) the slot is S1's partner: use S0.
    // (w0 == 2 pieces are addressed with slot S1 in plane 0 and S2 in plane 1; see the callers.)
#define KVQ_PAIR(K)                                                                                   \
    {                                                                                                 \
      constexpr int s0 = (w0 == 4) ? 0 : S1;                                                          \
      constexpr int q0 = pair_q<w0, s0, K>();                                                         \
      const uint32_t h0 = extract_pair<w0, s0, K>(pw.w[0]);                                           \
      constexpr float f0 = 1.0f / (float)(1 << q0);                                                   \
      if constexpr (np == 1) {                                                                        \
        constexpr float c0 = -(1024.0f * f0 + (float)off);                                           \
        half2v res = __builtin_elementwise_fma(as_h2(h0), half2v{(_Float16)f0, (_Float16)f0},          \
                                               half2v{(_Float16)c0, (_Float16)c0});                   \
        r[K] = as_u(res);                                                                             \
      } else if constexpr (np == 2) {                                                                 \
        constexpr int s1 = (w0 == 4) ? S1 : S2;                                                       \
        constexpr int q1 = pair_q<w1, s1, K>();                                                       \
        const uint32_t h1 = extract_pair<w1, s1, K>(pw.w[1]);                                         \
        constexpr float f1 = (float)(1 << sh1) / (float)(1 << q1);                                    \
        constexpr float c1 = -(1024.0f * (f0 + f1) + (float)off);                                     \
        half2v acc = __builtin_elementwise_fma(as_h2(h1), half2v{(_Float16)f1, (_Float16)f1},          \
                                               half2v{(_Float16)c1, (_Float16)c1});                   \
        acc = __builtin_elementwise_fma(as_h2(h0), half2v{(_Float16)f0, (_Float16)f0}, acc);           \
        r[K] = as_u(acc);                                                                             \
      } else {                                                                                        \
        constexpr int q1 = pair_q<w1, S1, K>();                                                       \
        constexpr int q2 = pair_q<w2, S2, K>();                                                       \
        const uint32_t h1 = extract_pair<w1, S1, K>(pw.w[1]);                                         \
        const uint32_t h2 = extract_pair<w2, S2, K>(pw.w[2]);                                         \
        constexpr float f1 = (float)(1 << sh1) / (float)(1 << q1);                                    \
        constexpr float f2 = (float)(1 << sh2) / (float)(1 << q2);                                    \
        constexpr float c12 = -(1024.0f * (f0 + f1) + (float)off);                                    \
        half2v t2 = as_h2(h2) - half2v{(_Float16)1024.0f, (_Float16)1024.0f};                         \
        half2v acc = __builtin_elementwise_fma(t2, half2v{(_Float16)f2, (_Float16)f2},                 \
                                               half2v{(_Float16)c12, (_Float16)c12});                 \
        acc = __builtin_elementwise_fma(as_h2(h1), half2v{(_Float16)f1, (_Float16)f1}, acc);           \
        acc = __builtin_elementwise_fma(as_h2(h0), half2v{(_Float16)f0, (_Float16)f0}, acc);           \
        r[K] = as_u(acc);                                                                             \
      }                                                                                               \
    }
    KVQ_PAIR(0)
    KVQ_PAIR(1)
    KVQ_PAIR(2)
    KVQ_PAIR(3)
#undef KVQ_PAIR
    return __builtin_bit_cast(half8, r);
  }
}

// Decode piece index `i` (block b for K, n-tile n for V) given the per-plane runs of words.
// run0 holds plane 0's words, run1 plane 1's, run2 plane 2's (indexed in 32-bit words).
template <int N, int I>
__device__ inline half8 decode_run_piece(const uint32_t* run0, const uint32_t* run1, const uint32_t* run2) {
  PieceWords pw;
  if constexpr (N == 8) {
    pw.w[0] = run0[2 * I];
    pw.w[1] = run0[2 * I + 1];
    pw.w[2] = 0;
    return decode_piece<8, 0, 0>(pw);
  } else {
    constexpr int w0 = Planes<N>::w[0];
    constexpr int w1 = Planes<N>::w[1];
    constexpr int w2 = Planes<N>::w[2];
    constexpr int per0 = 4 / w0;
    pw.w[0] = run0[I / per0];
    if constexpr (w0 == 4) {
      if constexpr (Planes<N>::n >= 2) pw.w[1] = run1[I / (4 / w1)];
      if constexpr (Planes<N>::n >= 3) pw.w[2] = run2[I / (4 / w2)];
      constexpr int s1 = (Planes<N>::n >= 2) ? I % (4 / (w1 ? w1 : 4)) : 0;
      constexpr int s2 = (Planes<N>::n >= 3) ? I % (4 / (w2 ? w2 : 4)) : 0;
      return decode_piece<N, s1, s2>(pw);
    } else {
      // w0 == 2 (N = 2 or 3): plane 0 slot = I % 2, plane 1 (w = 1) slot = I % 4
      if constexpr (Planes<N>::n >= 2) pw.w[1] = run1[I / 4];
      constexpr int s0 = I % 2;
      constexpr int s1 = (Planes<N>::n >= 2) ? I % 4 : 0;
      return decode_piece<N, s0, s1>(pw);
    }
  }
}

// ------------------------------------------------------------------ small helpers

__device__ inline float dpp_ror8(float x) {
  // lane i of each row of 16 receives lane (i + 8) % 16
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

__device__ inline float wave_max_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

template <int W>
__device__ inline void load_words(const uint8_t* p, uint32_t* dst, int n_words) {
  // n_words is a compile-time multiple of 2 or 4 at every call site
  if (n_words % 4 == 0) {
    for (int k = 0; k < n_words; k += 4) {
      u32x4 v = *(const u32x4*)(p + 4 * k);
      dst[k] = v[0]; dst[k + 1] = v[1]; dst[k + 2] = v[2]; dst[k + 3] = v[3];
    }
  } else {
    for (int k = 0; k < n_words; k += 2) {
      u32x2 v = *(const u32x2*)(p + 4 * k);
      dst[k] = v[0]; dst[k + 1] = v[1];
    }
  }
}

// ------------------------------------------------------------------ per-wave state

struct WaveState {
  floatx4 o[16];   // C[row = 4g + r][col = d16] per n-tile: rows 0-7 hi heads, 8-15 lo heads
  float m;         // running max (exp2 domain) of this lane's head
  float l;         // running sum of p over this lane's positions
};

// One 32-position tile of a qN_0 store (body, or the q8_0 ring).
//   krow(pos) gives the K row of a position; vt is the V tile; [lo, hi) the valid positions.
template <int NK, int NV>
__device__ inline void tile_quant(WaveState& st, const half8* qb, float qmul, const uint8_t* kbase, int row_k,
                                  bool ring, int R, const uint8_t* vt, int tile, int lo, int hi, bool lo_lane) {
  constexpr int D = 256, NB = 8, NT = 16;
  const int lane = threadIdx.x & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;
  constexpr int w0k = Planes<NK>::w[0], w1k = Planes<NK>::w[1], w2k = Planes<NK>::w[2];
  constexpr int w0v = Planes<NV>::w[0], w1v = Planes<NV>::w[1], w2v = Planes<NV>::w[2];

  // ---- scores for the two 16-position subtiles
  float sc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int pos = tile * kTile + 16 * s + m16;
    const uint8_t* row = kbase + (size_t)(ring ? pos % R : pos) * row_k;
    uint32_t k0[NB * w0k / 4 + 1], k1[(w1k ? NB * w1k / 4 : 1) + 1], k2[(w2k ? NB * w2k / 4 : 1) + 1];
    load_words<0>(row + g * NB * w0k, k0, NB * w0k / 4);
    if constexpr (w1k) load_words<0>(row + 4 * NB * w0k + g * NB * w1k, k1, NB * w1k / 4);
    if constexpr (w2k) load_words<0>(row + 4 * NB * (w0k + w1k) + g * NB * w2k, k2, NB * w2k / 4);
    // scales of rows 4g + r
    u32x4 dk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pr = tile * kTile + 16 * s + 4 * g + r;
      const uint8_t* rr = kbase + (size_t)(ring ? pr % R : pr) * row_k;
      dk[r] = *(const u32x4*)(rr + NB * 4 * NK);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[s][r] = 0.0f;
#define KVQ_QK(B)                                                                                 \
    {                                                                                             \
      half8 a = decode_run_piece<NK, B>(k0, k1, k2);                                              \
      floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[B], floatx4{0, 0, 0, 0}, 0, 0, 0);  \
      _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                             \
        const uint32_t wd = dk[r][B >> 1];                                                        \
        const float d = h2f((uint16_t)((B & 1) ? (wd >> 16) : (wd & 0xFFFF)));                    \
        sc[s][r] = fmaf(c[r], d, sc[s][r]);                                                       \
      }                                                                                           \
    }
    KVQ_QK(0) KVQ_QK(1) KVQ_QK(2) KVQ_QK(3) KVQ_QK(4) KVQ_QK(5) KVQ_QK(6) KVQ_QK(7)
#undef KVQ_QK
  }

  // ---- V codes and scales of this lane (positions T(g, i))
  uint32_t v0[NT * w0v / 4], v1[(w1v ? NT * w1v / 4 : 1)], v2[(w2v ? NT * w2v / 4 : 1)];
  {
    const int run0 = NT * w0v;        // bytes per lane
#pragma unroll
    for (int c = 0; c < run0 / 16; ++c) {
      u32x4 x = *(const u32x4*)(vt + c * 1024 + lane * 16);
      v0[4 * c] = x[0]; v0[4 * c + 1] = x[1]; v0[4 * c + 2] = x[2]; v0[4 * c + 3] = x[3];
    }
    if constexpr (w1v) {
      const uint8_t* p1 = vt + 64 * NT * w0v;
#pragma unroll
      for (int c = 0; c < NT * w1v / 16; ++c) {
        u32x4 x = *(const u32x4*)(p1 + c * 1024 + lane * 16);
        v1[4 * c] = x[0]; v1[4 * c + 1] = x[1]; v1[4 * c + 2] = x[2]; v1[4 * c + 3] = x[3];
      }
    }
    if constexpr (w2v) {
      const uint8_t* p2 = vt + 64 * NT * (w0v + w1v);
      u32x4 x = *(const u32x4*)(p2 + lane * 16);
      v2[0] = x[0]; v2[1] = x[1]; v2[2] = x[2]; v2[3] = x[3];
    }
  }
  u32x4 dv[8];
  {
    const uint8_t* sp = vt + 4 * D * NV;
#pragma unroll
    for (int i = 0; i < 8; ++i) dv[i] = *(const u32x4*)(sp + tile_pos(g, i) * NB * 2);
  }

  // ---- softmax update
  float x[8];
  float tmax = kNegBig;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float full = sc[s][r] + dpp_ror8(sc[s][r]);
      const int pos = tile * kTile + 16 * s + 4 * g + r;
      const float v = (pos >= lo && pos < hi) ? full * qmul : -INFINITY;
      x[4 * s + r] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = wave_max_16_32(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float p[8];
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    psum += p[i];
  }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int n = 0; n < NT; ++n) st.o[n] *= alpha;

  // ---- P.V: per block b, A = P * dv16 (hi rows / lo rows), B = V codes of n-tiles 2b, 2b+1
  const float kf = lo_lane ? 1.0f : 0.0f;
#define KVQ_PV(B)                                                                                   \
  {                                                                                                 \
    half8 a;                                                                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                 \
      const uint32_t wd = dv[i][B >> 1];                                                            \
      const float d = h2f((uint16_t)((B & 1) ? (wd >> 16) : (wd & 0xFFFF)));                        \
      const float xv = p[i] * d;                                                                    \
      const _Float16 h = (_Float16)xv;                                                              \
      const float y = fmaf(-kf, (float)h, xv);                                                      \
      a[i] = (_Float16)y;                                                                           \
    }                                                                                               \
    half8 b0 = decode_run_piece<NV, 2 * B>(v0, v1, v2);                                             \
    st.o[2 * B] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b0, st.o[2 * B], 0, 0, 0);              \
    half8 b1 = decode_run_piece<NV, 2 * B + 1>(v0, v1, v2);                                         \
    st.o[2 * B + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b1, st.o[2 * B + 1], 0, 0, 0);      \
  }
  KVQ_PV(0) KVQ_PV(1) KVQ_PV(2) KVQ_PV(3) KVQ_PV(4) KVQ_PV(5) KVQ_PV(6) KVQ_PV(7)
#undef KVQ_PV
}

// One 32-position tile of the bf16 tail ring.
__device__ inline void tile_bf16(WaveState& st, const bf16x8* qb, float qmul, const uint8_t* kring, int R,
                                 const uint8_t* vt, int tile, int lo, int hi, bool lo_lane) {
  constexpr int D = 256, NT = 16;
  const int lane = threadIdx.x & 63;
  const int m16 = lane & 15;
  const int g = lane >> 4;
  float sc[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int pos = tile * kTile + 16 * s + m16;
    const uint8_t* row = kring + (size_t)(pos % R) * (2 * D);
    floatx4 c = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      bf16x8 a = *(const bf16x8*)(row + (32 * b + 8 * g) * 2);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[b], c, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[s][r] = c[r];
  }
  bf16x8 vv[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) vv[n] = *(const bf16x8*)(vt + n * 1024 + lane * 16);

  float x[8];
  float tmax = kNegBig;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = tile * kTile + 16 * s + 4 * g + r;
      const float v = (pos >= lo && pos < hi) ? sc[s][r] * qmul : -INFINITY;
      x[4 * s + r] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = wave_max_16_32(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float psum = 0.0f;
  bf16x8 a;
  const float kf = lo_lane ? 1.0f : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_amdgcn_exp2f(x[i] - m_new);
    psum += p;
    const __bf16 h = (__bf16)p;
    const float y = fmaf(-kf, (float)h, p);
    a[i] = (__bf16)y;
  }
  st.l = st.l * alpha + psum;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    st.o[n] *= alpha;
    st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vv[n], st.o[n], 0, 0, 0);
  }
}

// ------------------------------------------------------------------ the split kernel

template <int NK, int NV>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int D = 256, NB = 8, NT = 16;
  __shared__ float s_o[4][kPartialHeads][D];
  __shared__ float s_ml[4][2][kPartialHeads];

  const int split = blockIdx.x;
  const int head = blockIdx.y;
  const int si = blockIdx.z;
  const DecodeSeq S = a.seqs[si];
  const int n_splits = S.n_body_splits + S.n_ring_splits;
  if (split >= n_splits) return;
  const Geometry& g = a.g;
  const bool is_ring = split >= S.n_body_splits;
  const int tail = g.tail_dtype;
  const int R = g.ring_slots;
  const uint8_t* slab = g.arena + S.slab;

  int tile_begin, tile_end, lo, hi;
  if (!is_ring) {
    const int body_tiles = (S.body_len + kTile - 1) / kTile;
    tile_begin = split * a.tiles_per_split;
    tile_end = min(body_tiles, tile_begin + a.tiles_per_split);
    lo = 0;
    hi = S.body_len;
  } else {
    const int rs = split - S.n_body_splits;
    const int ring_end = (S.len + kTile - 1) / kTile;
    tile_begin = S.ring_tile0 + rs * a.tiles_per_split;
    tile_end = min(ring_end, tile_begin + a.tiles_per_split);
    lo = S.body_len;
    hi = S.len;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
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
  if (is_ring && tail == 1) {
    bf16x8 qb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // columns 8-15 repeat heads 0-7 so the lo-part lanes see the same scores
      bf16x8 v = *(const bf16x8*)(qrow + 32 * b + 8 * gq);
      if (!head_ok) v = bf16x8{};
      qb[b] = v;
    }
    const float qmul = a.scale * kLog2e;
    const uint8_t* kring = slab + g.k_ring + (size_t)head * R * (2 * D);
    for (int t = tile_begin + wave; t < tile_end; t += 4) {
      const uint8_t* vt = slab + g.v_ring + ((size_t)head * (R / kTile) + ((t * kTile) % R) / kTile) * g.ring_tile_v;
      tile_bf16(st, qb, qmul, kring, R, vt, t, lo, hi, lo_lane);
    }
  } else {
    // exponent-shifted query (times KVarN sigma), split into fp16 hi (cols 0-7) and lo (cols 8-15)
    float xq[NB][8];
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      u32x4 raw = *(const u32x4*)(qrow + 32 * b + 8 * gq);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xq[b][2 * k] = __uint_as_float(raw[k] << 16);
        xq[b][2 * k + 1] = __uint_as_float(raw[k] & 0xFFFF0000u);
      }
      if (use_sigma) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xq[b][i] *= h2f(sig[32 * b + 8 * gq + i]);   // exact (8 + 11 bits)
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xq[b][i]));
    }
    amax = wave_max_16_32(amax);
    const int e = amax > 0.0f ? ilogbf(amax) - 14 : 0;
    half8 qb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xs = ldexpf(xq[b][i], -e);
        const _Float16 h = (_Float16)xs;
        const _Float16 l = (_Float16)(xs - (float)h);
        qb[b][i] = head_ok ? (lo_lane ? l : h) : (_Float16)0.0f;
      }
    }
    const float qmul = a.scale * kLog2e * ldexpf(1.0f, e);
    if (!is_ring) {
      const uint8_t* kbase = slab + g.k_body + (size_t)head * g.cap32 * g.row_k;
      for (int t = tile_begin + wave; t < tile_end; t += 4) {
        const uint8_t* vt = slab + g.v_body + ((size_t)head * (g.cap32 / kTile) + t) * g.tile_v;
        tile_quant<NK, NV>(st, qb, qmul, kbase, g.row_k, false, 1, vt, t, lo, hi, lo_lane);
      }
    } else {
      const uint8_t* kbase = slab + g.k_ring + (size_t)head * R * g.ring_row_k;
      for (int t = tile_begin + wave; t < tile_end; t += 4) {
        const uint8_t* vt = slab + g.v_ring + ((size_t)head * (R / kTile) + ((t * kTile) % R) / kTile) * g.ring_tile_v;
        tile_quant<8, 8>(st, qb, qmul, kbase, g.ring_row_k, true, R, vt, t, lo, hi, lo_lane);
      }
    }
  }

  // ---- wave epilogue: l over the lanes of a head; o = hi rows + lo rows
  float lsum = lo_lane ? 0.0f : st.l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) st.o[n][r] += __shfl_xor(st.o[n][r], 32);
  if (gq < 2) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][4 * gq + r][16 * n + m16] = st.o[n][r];
  }
  if (lane < 8) {
    s_ml[wave][0][lane] = st.m;
    s_ml[wave][1][lane] = lsum;
  }
  __syncthreads();

  // ---- merge the 4 waves and write the partial of this split
  float* part = a.partials + (((size_t)si * g.n_kv_heads + head) * a.max_splits + split) * (kPartialHeads * (D + 2));
  const float vs = (use_sigma) ? h2f(sig[D + tid]) : 1.0f;
  for (int h = 0; h < kPartialHeads; ++h) {
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_ml[w][0][h] - M);
      L += s_ml[w][1][h] * f;
      O += s_o[w][h][tid] * f;
    }
    part[2 * kPartialHeads + h * D + tid] = O * vs;
    if (tid == 0) {
      part[h] = M;
      part[kPartialHeads + h] = L;
    }
  }
}

// ------------------------------------------------------------------ combine

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int si = blockIdx.x / a.n_kv_heads;
  const int head = blockIdx.x % a.n_kv_heads;
  const int D = a.head_dim;
  const int ns = a.n_splits[si];
  const float* base = a.partials + ((size_t)si * a.n_kv_heads + head) * a.max_splits * (kPartialHeads * (D + 2));
  const size_t rec = kPartialHeads * (D + 2);
  for (int h = 0; h < a.group; ++h) {
    float M = kNegBig;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * rec + h]);
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
      float L = 0.0f, O = 0.0f;
      for (int s = 0; s < ns; ++s) {
        const float f = __builtin_amdgcn_exp2f(base[s * rec + h] - M);
        L += base[s * rec + kPartialHeads + h] * f;
        O += base[s * rec + 2 * kPartialHeads + h * D + c] * f;
      }
      a.out[((size_t)si * a.n_q_heads + head * a.group + h) * D + c] = O / L;
    }
  }
}

template <int NK, int NV>
hipError_t launch_decode_t(const DecodeArgs& a, int grid_x, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<NK, NV>), dim3(grid_x, a.g.n_kv_heads, a.n_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int grid_x, hipStream_t s) {
  const int nk = a.g.k_bits, nv = a.g.v_bits;
#define KVQ_CASE(K, V) if (nk == K && nv == V) return launch_decode_t<K, V>(a, grid_x, s);
#define KVQ_ROW(K) KVQ_CASE(K, 2) KVQ_CASE(K, 3) KVQ_CASE(K, 4) KVQ_CASE(K, 5) KVQ_CASE(K, 6) KVQ_CASE(K, 7) KVQ_CASE(K, 8)
  KVQ_ROW(2) KVQ_ROW(3) KVQ_ROW(4) KVQ_ROW(5) KVQ_ROW(6) KVQ_ROW(7) KVQ_ROW(8)
#undef KVQ_ROW
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.n_seqs * a.n_kv_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse(const SparseArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvq
