// Operand helpers shared by the decode kernels: vector types, the compile-time plane description of an
// N-bit code, exact fp16 decoding of packed codes (the "1024 + value" form for P.V operands, and bit planes
// as fp16 denormals for QK operands), and cross-row lane reductions of gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
__device__ inline uint32_t extract_pair(uint32_t word, uint32_t magic) {
  constexpr int q = pair_offset(W, SLOT, K) - pair_pre_shift(W, SLOT, K);
  constexpr uint32_t m = ((1u << W) - 1) << q;
  constexpr uint32_t mask = m | (m << 16);
  constexpr int s = pair_pre_shift(W, SLOT, K);
  return ((word >> s) & mask) | magic;      // one v_and_or_b32 (mask from an SGPR, magic from a VGPR)
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
__device__ inline half8 decode_piece(const PieceWords& pw, uint32_t magic) {
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
      const uint32_t h0 = extract_pair<w0, s0, K>(pw.w[0], magic);                                           \
      constexpr float f0 = 1.0f / (float)(1 << q0);                                                   \
      if constexpr (np == 1) {                                                                        \
        constexpr float c0 = -(1024.0f * f0 + (float)off);                                           \
        half2v res = __builtin_elementwise_fma(as_h2(h0), half2v{(_Float16)f0, (_Float16)f0},          \
                                               half2v{(_Float16)c0, (_Float16)c0});                   \
        r[K] = as_u(res);                                                                             \
      } else if constexpr (np == 2) {                                                                 \
        constexpr int s1 = (w0 == 4) ? S1 : S2;                                                       \
        constexpr int q1 = pair_q<w1, s1, K>();                                                       \
        const uint32_t h1 = extract_pair<w1, s1, K>(pw.w[1], magic);                                         \
        constexpr float f1 = (float)(1 << sh1) / (float)(1 << q1);                                    \
        constexpr float c1 = -(1024.0f * (f0 + f1) + (float)off);                                     \
        half2v acc = __builtin_elementwise_fma(as_h2(h1), half2v{(_Float16)f1, (_Float16)f1},          \
                                               half2v{(_Float16)c1, (_Float16)c1});                   \
        acc = __builtin_elementwise_fma(as_h2(h0), half2v{(_Float16)f0, (_Float16)f0}, acc);           \
        r[K] = as_u(acc);                                                                             \
      } else {                                                                                        \
        constexpr int q1 = pair_q<w1, S1, K>();                                                       \
        constexpr int q2 = pair_q<w2, S2, K>();                                                       \
        const uint32_t h1 = extract_pair<w1, S1, K>(pw.w[1], magic);                                         \
        const uint32_t h2 = extract_pair<w2, S2, K>(pw.w[2], magic);                                         \
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
__device__ inline half8 decode_run_piece(const uint32_t* run0, const uint32_t* run1, const uint32_t* run2,
                                         uint32_t magic) {
  PieceWords pw;
  if constexpr (N == 8) {
    pw.w[0] = run0[2 * I];
    pw.w[1] = run0[2 * I + 1];
    pw.w[2] = 0;
    return decode_piece<8, 0, 0>(pw, magic);
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
      return decode_piece<N, s1, s2>(pw, magic);
    } else {
      // w0 == 2 (N = 2 or 3): plane 0 slot = I % 2, plane 1 (w = 1) slot = I % 4
      if constexpr (Planes<N>::n >= 2) pw.w[1] = run1[I / 4];
      constexpr int s0 = I % 2;
      constexpr int s1 = (Planes<N>::n >= 2) ? I % 4 : 0;
      return decode_piece<N, s0, s1>(pw, magic);
    }
  }
}

// ------------------------------------------------------------------ K planes as fp16 denormals
//
// For QK each bit plane of a K piece goes to the MFMA on its own, as fp16 denormal numbers: an AND of
// the plane word leaves the field of pair k in both 16-bit halves at bit offset q_k, i.e. the half is the
// exact denormal field * 2^(q_k - 24). The query operand of that plane carries the compensating weight
// 2^(plane shift - q_k) per element, so the plane MFMAs add up to 2^-24 * sum(u * q) for the biased code u;
// the bias is removed by one more MFMA of a constant operand (-2^(N-1) * 2^(q_k - 24), also exact) with
// the plane-0 query operand. gfx950's MFMA treats fp16 denormal inputs exactly. Fields at bits 8 and above are shifted down by 8 first so that every field stays in the
// mantissa (bits 0-9).

// Bit offset q of the field of element i after the extraction below (plane width W, piece slot SLOT).
__device__ inline int dn_bitpos(int w, int slot, int i) {
  const int k = i >> 1;
  return w == 8 ? 0 : w == 4 ? 4 * (k & 1) : w == 2 ? 2 * k : 4 * (slot & 1) + k;
}

template <int W, int SLOT>
__device__ inline half8 dn_extract(uint32_t word) {
  u32x4 r;
  if constexpr (W == 4) {
    const uint32_t w8 = word >> 8;
    r[0] = word & 0x000F000Fu;
    r[1] = word & 0x00F000F0u;
    r[2] = w8 & 0x000F000Fu;
    r[3] = w8 & 0x00F000F0u;
  } else if constexpr (W == 2) {
    const uint32_t ws = SLOT ? word >> 8 : word;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = ws & (0x00030003u << (2 * k));
  } else {
    const uint32_t ws = SLOT >= 2 ? word >> 8 : word;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = ws & (0x00010001u << (4 * (SLOT & 1) + k));
  }
  return __builtin_bit_cast(half8, r);
}

// The plane operands of K piece B (block B) from the lane's runs of plane words.
template <int N> struct KPlanes { half8 a[Planes<N>::n]; };

template <int N, int B>
__device__ inline void dn_piece(const uint32_t* run0, const uint32_t* run1, const uint32_t* run2, KPlanes<N>& kp) {
  if constexpr (N == 8) {
    // bytes -> halves (0x00, byte): the byte itself as a denormal
    const uint32_t lo = run0[2 * B], hi = run0[2 * B + 1];
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(0u, lo, 0x0C010C00u);
    r[1] = __builtin_amdgcn_perm(0u, lo, 0x0C030C02u);
    r[2] = __builtin_amdgcn_perm(0u, hi, 0x0C010C00u);
    r[3] = __builtin_amdgcn_perm(0u, hi, 0x0C030C02u);
    kp.a[0] = __builtin_bit_cast(half8, r);
  } else {
    constexpr int w0 = Planes<N>::w[0], w1 = Planes<N>::w[1], w2 = Planes<N>::w[2];
    kp.a[0] = dn_extract<w0, B % (4 / w0)>(run0[(B * w0) / 4]);
    if constexpr (Planes<N>::n >= 2) kp.a[1] = dn_extract<w1, B % (4 / w1)>(run1[(B * w1) / 4]);
    if constexpr (Planes<N>::n >= 3) kp.a[2] = dn_extract<w2, B % (4 / w2)>(run2[(B * w2) / 4]);
  }
}

// ------------------------------------------------------------------ small helpers

__device__ inline float dpp_ror8(float x) {
  // lane i of each row of 16 receives lane (i + 8) % 16
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// Reductions across the four 16-lane rows of the wave with gfx950's lane-swap instructions, without LDS
// traffic: with both operands equal, v_permlane16_swap returns (rows 0,0,2,2) and (rows 1,1,3,3) of x, and
// v_permlane32_swap returns (lanes 0-31 twice) and (lanes 32-63 twice), so combining the two results gives
// x op x[lane ^ 16] (or ^ 32) in every lane.
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float wave_max_16_32(float x) { return max_xor32(max_xor16(x)); }

// Cache rows are read once per decode call: streaming (nontemporal) loads keep them from displacing
// other lines and sustain a much higher read rate on gfx950 than ordinary loads.
__device__ inline u32x4 ldnt(const uint8_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }


// ------------------------------------------------------------------ per-wave attention state

struct WaveState {
  floatx4 o[16];   // C[row = 4g + r][col = d16] per n-tile: rows 0-7 hi heads, 8-15 lo heads
  float m;         // running max (exp2 domain) of this lane's head
  float l;         // running sum of p over this lane's positions
};

__device__ inline float lo_h(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ inline float hi_h(uint32_t w) { return (float)as_h2(w)[1]; }

// Online-softmax update for this lane's 8 scores x[] (exp2 domain, -inf for masked positions); returns p[].
// The scores are exponentiated against a reference max that moves only when some score of the wave exceeds it
// by more than kLazy: until then p <= 2^kLazy, well inside the range of the fp32 accumulators and of the fp16 /
// bf16 P.V operands, and the accumulators need no rescale (the split merge uses whatever reference a partial
// carries).
constexpr float kLazy = 8.0f;

__device__ inline void softmax_update(WaveState& st, const float* x, float* p) {
  float tmax = kNegBig;
#pragma unroll
  for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
  tmax = wave_max_16_32(tmax);
  if (__builtin_amdgcn_ballot_w64(tmax > st.m + kLazy)) {
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
    // The accumulator rows of lane (g, m16) are rows 4g..4g+3 of the P.V tile, i.e. heads 4g..4g+3 (hi parts for
    // g < 2, lo parts for g >= 2), not the lane's own score column m16: take those heads' factors from the lanes
    // of this 16-lane row that hold columns 4g..4g+3.
    const int lane = threadIdx.x & 63;
    const int src = (lane & 48) + ((lane >> 4) << 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((src + r) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
      for (int n = 0; n < 16; ++n) st.o[n][r] *= ar;
    }
  }
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(x[i] - st.m);
    psum += p[i];
  }
  st.l += psum;
}

}  // namespace
}  // namespace kvq
