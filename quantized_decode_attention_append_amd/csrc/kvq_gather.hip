// Gather decode: attention over an explicit list of positions of a row-layout cache (sparse decode of a
// QSA layer, offload page: the layer reads only the main-KV rows at the positions its indexer chose), and
// over all positions of a row-layout cache (dense decode with KVQ_LAYOUT_ROWS, list = 0..len-1).
//
// Every listed position is one K row and one V row, so the bytes read are exactly budget x row bytes.
// The work is small (a budget of 2048 positions is ~2 MB per layer) and latency-bound, so the kernel is
// plain VALU arithmetic in fp32; no tile staging:
//
// * grid (split, KV head, sequence); a work-group of 4 waves owns a contiguous range of list entries and
//   emits one partial (m, l, o) per query head of the group, merged by the same combine kernel as the
//   dense path;
// * a wave takes 16 list entries at a time. For QK, lane (p = lane & 15, j = lane >> 4) reads the pieces
//   (j, b = 0..7) of entry p's K row (channels 32b + 8j + i, contiguous in the row) and forms the 8 heads'
//   partial dot products with the query read from LDS; the 4 partial sums of a position are added by lane
//   shuffles;
// * online softmax in exp2 form (wave-wide max per head);
// * for P.V, lane c owns channels 4c..4c+3 of all 8 heads; for each of the 16 positions the weights are
//   broadcast with readlane and the lane decodes its 4 codes of that position's V row.
// Rows in the tail ring (positions >= body_len) are read as q8_0 or bf16 rows; KVarN scales apply to body
// rows only (K through the query, V per position).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGroup = 16;    // list entries per wave step
constexpr int kWaves = 4;

__device__ inline float f16f(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }
__device__ inline float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Compile-time plane description of an N-bit code (least significant plane first).
template <int N> struct PL;
template <> struct PL<2> { static constexpr int n = 1, w0 = 2, w1 = 0, w2 = 0, s1 = 0, s2 = 0; };
template <> struct PL<3> { static constexpr int n = 2, w0 = 2, w1 = 1, w2 = 0, s1 = 2, s2 = 0; };
template <> struct PL<4> { static constexpr int n = 1, w0 = 4, w1 = 0, w2 = 0, s1 = 0, s2 = 0; };
template <> struct PL<5> { static constexpr int n = 2, w0 = 4, w1 = 1, w2 = 0, s1 = 4, s2 = 0; };
template <> struct PL<6> { static constexpr int n = 2, w0 = 4, w1 = 2, w2 = 0, s1 = 4, s2 = 0; };
template <> struct PL<7> { static constexpr int n = 3, w0 = 4, w1 = 2, w2 = 1, s1 = 4, s2 = 6; };
template <> struct PL<8> { static constexpr int n = 1, w0 = 8, w1 = 0, w2 = 0, s1 = 0, s2 = 0; };

// Element i of piece `piece` (index j*NB + b within a plane of width w) of a row plane, given the plane's
// 32-bit words starting at `words` (the word holding the piece is words[piece * w / 4]).
template <int W>
__device__ inline uint32_t piece_elem(uint32_t word, int piece, int i) {
  if constexpr (W == 8) {
    return (word >> (8 * (i & 3))) & 0xFFu;   // word = bytes 4*(i/4).. of the piece
  } else {
    const int slot = piece % (4 / W);
    return (word >> (16 * (i & 1) + 4 * W * slot + W * (i >> 1))) & ((1u << W) - 1);
  }
}

// ---- QK side: the lane's 64 channels (pieces (j, b), b = 0..7) of one row

// Raw words of the lane's part of one row. Body/q8 rows: per plane the run of NB pieces for lane group j,
// then the 8 fp16 block scales. bf16 rows: 8 x 8 channels.
struct KRaw {
  uint32_t w[32];
};

template <int N>
__device__ inline void load_k_qrow(KRaw& r, const uint8_t* row, int j) {
  constexpr int NB = 8;
  using P = PL<N>;
  // plane 0 run: NB * w0 bytes at j * NB * w0
  constexpr int n0 = NB * P::w0 / 4, n1 = NB * P::w1 / 4, n2 = NB * P::w2 / 4;
  const uint8_t* p0 = row + j * NB * P::w0;
#pragma unroll
  for (int k = 0; k < n0; k += (n0 >= 4 ? 4 : 2)) {
    if constexpr (n0 >= 4) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(p0 + 4 * k));
      r.w[k] = v[0]; r.w[k + 1] = v[1]; r.w[k + 2] = v[2]; r.w[k + 3] = v[3];
    } else {
      const u32x2 v = __builtin_nontemporal_load((const u32x2*)(p0 + 4 * k));
      r.w[k] = v[0]; r.w[k + 1] = v[1];
    }
  }
  if constexpr (P::n >= 2) {
    const uint8_t* p1 = row + 4 * NB * P::w0 + j * NB * P::w1;
#pragma unroll
    for (int k = 0; k < n1; k += (n1 >= 4 ? 4 : 2)) {
      if constexpr (n1 >= 4) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)(p1 + 4 * k));
        r.w[16 + k] = v[0]; r.w[16 + k + 1] = v[1]; r.w[16 + k + 2] = v[2]; r.w[16 + k + 3] = v[3];
      } else {
        const u32x2 v = __builtin_nontemporal_load((const u32x2*)(p1 + 4 * k));
        r.w[16 + k] = v[0]; r.w[16 + k + 1] = v[1];
      }
    }
  }
  if constexpr (P::n >= 3) {
    const uint8_t* p2 = row + 4 * NB * (P::w0 + P::w1) + j * NB * P::w2;
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p2);
    r.w[24] = v[0]; r.w[25] = v[1];
  }
  const u32x4 sc = __builtin_nontemporal_load((const u32x4*)(row + 4 * NB * N));
  r.w[28] = sc[0]; r.w[29] = sc[1]; r.w[30] = sc[2]; r.w[31] = sc[3];
}

// The 8 values of block b (channels 32b + 8j + i) of a qN_0 row part loaded by load_k_qrow.
template <int N>
__device__ inline void k_block_values(const KRaw& r, int j, int b, float* x) {
  constexpr int NB = 8;
  using P = PL<N>;
  const float d = f16f(r.w[28 + (b >> 1)] >> (16 * (b & 1)));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t u;
    if constexpr (N == 8) {
      u = piece_elem<8>(r.w[2 * b + (i >> 2)], 0, i);
    } else {
      const int pc = j * NB + b;   // piece index in the plane; the lane's run starts at piece j * NB
      u = piece_elem<P::w0>(r.w[(b * P::w0) / 4], pc, i);
      if constexpr (P::n >= 2) u |= piece_elem<P::w1>(r.w[16 + (b * P::w1) / 4], pc, i) << P::s1;
      if constexpr (P::n >= 3) u |= piece_elem<P::w2>(r.w[24 + (b * P::w2) / 4], pc, i) << P::s2;
    }
    x[i] = (float)((int)u - (1 << (N - 1))) * d;   // exact: integer code times an fp16 scale
  }
}

__device__ inline void load_k_bf16(KRaw& r, const uint8_t* row, int j) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(row + (32 * b + 8 * j) * 2));
    r.w[4 * b] = v[0]; r.w[4 * b + 1] = v[1]; r.w[4 * b + 2] = v[2]; r.w[4 * b + 3] = v[3];
  }
}

// Partial scores of the 8 heads over the lane's 64 channels of one qN_0 row (qt: query [channel][head]).
template <int N>
__device__ inline void qk_qrow(const KRaw& kr, int j, const float (*qt)[kPartialHeads], float* acc) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    float x[8];
    k_block_values<N>(kr, j, b, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* qc = qt[32 * b + 8 * j + i];
#pragma unroll
      for (int h = 0; h < kPartialHeads; ++h) acc[h] = fmaf(x[i], qc[h], acc[h]);
    }
    __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounds the live query values
  }
}

__device__ inline void qk_bf16(const KRaw& kr, int j, const float (*qt)[kPartialHeads], float* acc) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = bf16f((kr.w[4 * b + (i >> 1)] >> (16 * (i & 1))) & 0xFFFFu);
      const float* qc = qt[32 * b + 8 * j + i];
#pragma unroll
      for (int h = 0; h < kPartialHeads; ++h) acc[h] = fmaf(x, qc[h], acc[h]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- P.V side: channels 4c..4c+3 of one V row

struct VRaw {
  uint32_t w[4];   // one word per plane (w <= 3 planes) + the block scale in w[3] (bf16: w[0..1])
};

template <int N>
__device__ inline void load_v_qrow(VRaw& r, const uint8_t* row, int c) {
  constexpr int NB = 8;
  using P = PL<N>;
  const int b = c >> 3, j = (c & 7) >> 1;
  const int pc = j * NB + b;
  if constexpr (N == 8) {
    r.w[0] = __builtin_nontemporal_load((const uint32_t*)(row + pc * 8 + 4 * (c & 1)));
  } else {
    r.w[0] = __builtin_nontemporal_load((const uint32_t*)(row + 4 * ((pc * P::w0) / 4)));
    if constexpr (P::n >= 2)
      r.w[1] = __builtin_nontemporal_load((const uint32_t*)(row + 4 * NB * P::w0 + 4 * ((pc * P::w1) / 4)));
    if constexpr (P::n >= 3)
      r.w[2] = __builtin_nontemporal_load(
          (const uint32_t*)(row + 4 * NB * (P::w0 + P::w1) + 4 * ((pc * P::w2) / 4)));
  }
  r.w[3] = __builtin_nontemporal_load((const uint16_t*)(row + 4 * NB * N + 2 * b));
}

template <int N>
__device__ inline void v_values(const VRaw& r, int c, float* v) {
  constexpr int NB = 8;
  using P = PL<N>;
  const int b = c >> 3, j = (c & 7) >> 1, i0 = 4 * (c & 1);
  const int pc = j * NB + b;
  const float d = f16f(r.w[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t u;
    if constexpr (N == 8) {
      u = (r.w[0] >> (8 * k)) & 0xFFu;
    } else {
      u = piece_elem<P::w0>(r.w[0], pc, i0 + k);
      if constexpr (P::n >= 2) u |= piece_elem<P::w1>(r.w[1], pc, i0 + k) << P::s1;
      if constexpr (P::n >= 3) u |= piece_elem<P::w2>(r.w[2], pc, i0 + k) << P::s2;
    }
    v[k] = (float)((int)u - (1 << (N - 1))) * d;
  }
}

// ---- the kernel

template <int NK, int NV>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int D = 256, NB = 8, G = kPartialHeads;
  __shared__ float s_q[2][D][G];               // [plain, times KVarN sigma_K][channel][head]
  __shared__ float s_o[kWaves][G][D];
  __shared__ float s_ml[kWaves][2][G];

  const Geometry& g = a.g;
  int rem = blockIdx.x, si = 0;
  for (;;) {
    const int n = g.n_kv_heads * a.seqs[si].n_splits;
    if (rem < n || si + 1 >= a.n_seqs) break;
    rem -= n;
    ++si;
  }
  const GatherSeq S = a.seqs[si];
  const int head = rem / S.n_splits;
  const int split = rem % S.n_splits;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = g.ring_slots;
  const uint8_t* slab = g.arena + S.slab;
  const bool kvarn = g.kvarn != 0;
  const uint16_t* sig = (const uint16_t*)(slab + g.sigma) + (size_t)head * 2 * D;

  // query of the group's heads (and times sigma_K for body rows), [channel][head] in LDS: thread (h, c0) reads
  // 8 channels of head h with one 16-byte load (one round trip for the whole work-group)
  {
    const int h = tid >> 5, c0 = 8 * (tid & 31);
    u32x4 qw = {0u, 0u, 0u, 0u};
    if (h < a.group) qw = *(const u32x4*)(a.q + ((size_t)si * a.n_q_heads + head * a.group + h) * D + c0);
    u32x4 sw = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};   // fp16 1.0
    if (kvarn) sw = *(const u32x4*)(sig + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float qv = bf16f((qw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      s_q[0][c0 + i][h] = qv;
      s_q[1][c0 + i][h] = qv * f16f((sw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);   // exact (8 + 11 bits)
    }
  }
  float sv[4];   // sigma_V of this lane's P.V channels
  {
    u32x2 vw = {0x3C003C00u, 0x3C003C00u};
    if (kvarn) vw = *(const u32x2*)(sig + D + 4 * lane);
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[k] = f16f((vw[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
  }
  __syncthreads();

  const int ib = (int)((long)split * S.n_list / S.n_splits);
  const int ie = (int)((long)(split + 1) * S.n_list / S.n_splits);
  const int p16 = lane & 15, j = lane >> 4;
  const float qmul = a.scale * kLog2e;
  const uint8_t* kbody = slab + g.k_body + (size_t)head * g.cap32 * g.row_k;
  const uint8_t* vbody = slab + g.v_body + (size_t)head * g.cap32 * g.row_v;
  const uint8_t* kring = slab + g.k_ring + (size_t)head * R * g.ring_row_k;
  const uint8_t* vring = slab + g.v_ring + (size_t)head * R * g.ring_row_v;
  const int32_t* plist = a.positions ? a.positions + (size_t)si * a.pos_stride : nullptr;

  float m[G], l[G], o[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[h][k] = 0.0f;
  }

  for (int g0 = ib + kGroup * wave; g0 < ie; g0 += kGroup * kWaves) {
    // ---- this lane's list entry (p16) and its source
    const int idx = g0 + p16;
    int pos = -1;
    if (idx < ie) pos = plist ? plist[idx] : idx;
    const bool valid = pos >= 0 && pos < S.len;
    const bool body = valid && pos < S.body_len;
    // ---- K part of the entry's row
    KRaw kr;
    if (body) {
      load_k_qrow<NK>(kr, kbody + (size_t)pos * g.row_k, j);
    } else if (valid) {
      if (g.tail_dtype == 2) load_k_qrow<8>(kr, kring + (size_t)(pos % R) * g.ring_row_k, j);
      else load_k_bf16(kr, kring + (size_t)(pos % R) * g.ring_row_k, j);
    }
    // ---- V loads for the 16 entries (lane = channel group), issued before the QK arithmetic
    VRaw vr[kGroup];
    uint32_t vmask = 0, bmask = 0;
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      const int pt = __builtin_amdgcn_readlane(pos, t);
      const bool vt = pt >= 0 && pt < S.len;
      if (vt) {
        vmask |= 1u << t;
        if (pt < S.body_len) {
          bmask |= 1u << t;
          load_v_qrow<NV>(vr[t], vbody + (size_t)pt * g.row_v, lane);
        } else if (g.tail_dtype == 2) {
          load_v_qrow<8>(vr[t], vring + (size_t)(pt % R) * g.ring_row_v, lane);
        } else {
          const u32x2 x = __builtin_nontemporal_load((const u32x2*)(vring + (size_t)(pt % R) * g.ring_row_v + 8 * lane));
          vr[t].w[0] = x[0];
          vr[t].w[1] = x[1];
        }
      }
    }
    // ---- scores: partial dot products over the lane's 64 channels, summed over the 4 lane groups
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;
    // (one path per row source, so that each path is straight-line code)
    if (body) qk_qrow<NK>(kr, j, s_q[1], acc);
    else if (valid && g.tail_dtype == 2) qk_qrow<8>(kr, j, s_q[0], acc);
    else if (valid) qk_bf16(kr, j, s_q[0], acc);
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc = acc[h] + __shfl_xor(acc[h], 16);
      sc += __shfl_xor(sc, 32);
      sc = valid ? sc * qmul : -INFINITY;
      float mx = sc;
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
      const float m_new = fmaxf(m[h], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
      m[h] = m_new;
      p[h] = __builtin_amdgcn_exp2f(sc - m_new);
      l[h] = l[h] * alpha + (j == 0 ? p[h] : 0.0f);
#pragma unroll
      for (int k = 0; k < 4; ++k) o[h][k] *= alpha;
    }
    // ---- P.V for the 16 entries
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      if (!(vmask & (1u << t))) continue;
      float v[4];
      if (bmask & (1u << t)) {
        v_values<NV>(vr[t], lane, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] *= sv[k];
      } else if (g.tail_dtype == 2) {
        v_values<8>(vr[t], lane, v);
      } else {
        v[0] = bf16f(vr[t].w[0] & 0xFFFFu);
        v[1] = bf16f(vr[t].w[0] >> 16);
        v[2] = bf16f(vr[t].w[1] & 0xFFFFu);
        v[3] = bf16f(vr[t].w[1] >> 16);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[h]), t));   // entry t
#pragma unroll
        for (int k = 0; k < 4; ++k) o[h][k] = fmaf(ph, v[k], o[h][k]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- wave partials to LDS, then the work-group merge
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ls = l[h];
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) ls += __shfl_xor(ls, o2);
    if (lane == 0) {
      s_ml[wave][0][h] = m[h];
      s_ml[wave][1][h] = ls;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) s_o[wave][h][4 * lane + k] = o[h][k];
  }
  __syncthreads();
  float* part = a.partials + (((size_t)si * g.n_kv_heads + head) * a.max_splits + split) * (G * (D + 2));
  const int c = tid;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_ml[w][0][h] - M);
      L += s_ml[w][1][h] * f;
      O += s_o[w][h][c] * f;
    }
    part[2 * G + h * D + c] = O;
    if (c == 0) {
      part[h] = M;
      part[G + h] = L;
    }
  }
}

template <int NK, int NV>
hipError_t launch_gather_t(const GatherArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(gather_kernel<NK, NV>, dim3(grid_x), dim3(256), s, e0, e1, a);
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int nk = a.g.k_bits, nv = a.g.v_bits;
#define KVQ_CASE(K, V) if (nk == K && nv == V) return launch_gather_t<K, V>(a, grid_x, s, e0, e1);
#define KVQ_ROW(K) KVQ_CASE(K, 2) KVQ_CASE(K, 3) KVQ_CASE(K, 4) KVQ_CASE(K, 5) KVQ_CASE(K, 6) KVQ_CASE(K, 7) KVQ_CASE(K, 8)
  KVQ_ROW(2) KVQ_ROW(3) KVQ_ROW(4) KVQ_ROW(5) KVQ_ROW(6) KVQ_ROW(7) KVQ_ROW(8)
#undef KVQ_ROW
#undef KVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
