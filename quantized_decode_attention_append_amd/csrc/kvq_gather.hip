// Gather decode: attention over an explicit list of positions of a row-layout cache (sparse decode of a
// QSA layer, offload page: the layer reads only the main-KV rows at the positions its indexer chose), and
// over all positions of a row-layout cache (dense decode with KVQ_LAYOUT_ROWS, list = 0..len-1).
//
// Every listed position is one K row and one V row, so the bytes read are exactly budget x row bytes.
// A budget of 2048 positions is ~2 MB per layer: the call is latency-bound, and what sets its time is the
// length of one wave's instruction stream. So:
//
// * grid (split, KV head, sequence); a work-group of 4 waves (one per SIMD) owns a contiguous range of list entries and
//   emits one partial (m, l, o) per query head of the group, merged by the same combine kernel as the
//   dense path;
// * a wave takes 16 list entries at a time. Lane (j = lane >> 4, e = lane & 15) loads the pieces (j, b),
//   b = 0..7, of entry e's K row (channels 32b + 8j + i, contiguous in the row): that is the B operand of
//   a 16x16x32 MFMA with the entries as columns, so QK is one MFMA per K bit plane and block, with the
//   codes as exact fp16 denormals and the query as A operand (rows 0-7: fp16 hi parts of the 8 heads of
//   the group, rows 8-15: lo parts, exponent-shifted and weighted per plane), scaled per (entry, block)
//   in fp32, the same scheme as the dense kernel;
// * online softmax in exp2 form (maximum over the 16 entries by DPP row operations); the weights go
//   through LDS to every lane;
// * for P.V, lane c owns channels 4c..4c+3 of all 8 heads and decodes its 4 codes of each entry's V row.
// Rows in the tail ring (positions >= body_len) are read as q8_0 rows (a second query operand without the
// KVarN scale), f16 rows (fp16 MFMA on the values with that operand) or bf16 rows (bf16 MFMA); KVarN scales apply to body rows only (K through the query, V per
// position).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"
#include "kvq_mfma.h"
#include "kvq_write.h"

namespace kvq {
namespace {

constexpr int kGroup = 16;    // list entries per wave step
constexpr int kGWaves = kGatherWaves;
static_assert(64 * kGWaves == 256, "the fused append gives each thread one channel of K and V");
static_assert(2 * (32 * 8 + 16) / 16 <= 64 * kGWaves, "one 16-byte store per thread covers both row images");
constexpr int kImgRow = 288;   // bytes per LDS row image (a q8_0 row is 272)

__device__ inline float f16f(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }
__device__ inline float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Element i of piece `piece` of a row plane of width W < 8, given the 32-bit word holding the piece.
template <int W>
__device__ inline uint32_t piece_elem(uint32_t word, int piece, int i) {
  const int slot = piece % (4 / W);
  return (word >> (16 * (i & 1) + 4 * W * slot + W * (i >> 1))) & ((1u << W) - 1);
}

// Maximum / sum over the 16 lanes of a row (DPP: swaps within quads, then rotations by 4 and 8).
#define KVQ_DPP(x, c) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), c, 0xF, 0xF, false))
__device__ inline float row16_max(float x) {
  x = fmaxf(x, KVQ_DPP(x, 0xB1));    // quad_perm(1, 0, 3, 2)
  x = fmaxf(x, KVQ_DPP(x, 0x4E));    // quad_perm(2, 3, 0, 1)
  x = fmaxf(x, KVQ_DPP(x, 0x124));   // row_ror 4
  x = fmaxf(x, KVQ_DPP(x, 0x128));   // row_ror 8
  return x;
}
__device__ inline float row16_sum(float x) {
  x += KVQ_DPP(x, 0xB1);
  x += KVQ_DPP(x, 0x4E);
  x += KVQ_DPP(x, 0x124);
  x += KVQ_DPP(x, 0x128);
  return x;
}
#undef KVQ_DPP

// ---- K side: the lane's 64 channels (pieces (j, b), b = 0..7) of one row

// Raw words of the lane's part of one row. qN_0 rows: per plane the run of 8 pieces of lane group j (plane 0
// at w[0..], plane 1 at w[16..], plane 2 at w[24..]), then the row's 8 fp16 block scales at w[28..31].
// bf16 rows: 8 x 8 channels at w[0..31].
struct KRaw {
  uint32_t w[32];
};

template <int N>
__device__ inline void load_k_qrow(KRaw& r, const uint8_t* row, int j) {
  constexpr int NB = 8;
  using P = Planes<N>;
  constexpr int w0 = P::w[0], w1 = P::w[1], w2 = P::w[2];
  constexpr int n0 = NB * w0 / 4, n1 = NB * w1 / 4;
  const uint8_t* p0 = row + j * NB * w0;
#pragma unroll
  for (int k = 0; k < n0; k += (n0 >= 4 ? 4 : 2)) {
    if constexpr (n0 >= 4) {
      const u32x4 v = *((const u32x4*)(p0 + 4 * k));
      r.w[k] = v[0]; r.w[k + 1] = v[1]; r.w[k + 2] = v[2]; r.w[k + 3] = v[3];
    } else {
      const u32x2 v = *((const u32x2*)(p0 + 4 * k));
      r.w[k] = v[0]; r.w[k + 1] = v[1];
    }
  }
  if constexpr (P::n >= 2) {
    const uint8_t* p1 = row + 4 * NB * w0 + j * NB * w1;
#pragma unroll
    for (int k = 0; k < n1; k += (n1 >= 4 ? 4 : 2)) {
      if constexpr (n1 >= 4) {
        const u32x4 v = *((const u32x4*)(p1 + 4 * k));
        r.w[16 + k] = v[0]; r.w[16 + k + 1] = v[1]; r.w[16 + k + 2] = v[2]; r.w[16 + k + 3] = v[3];
      } else {
        const u32x2 v = *((const u32x2*)(p1 + 4 * k));
        r.w[16 + k] = v[0]; r.w[16 + k + 1] = v[1];
      }
    }
  }
  if constexpr (P::n >= 3) {
    const u32x2 v = *((const u32x2*)(row + 4 * NB * (w0 + w1) + j * NB * w2));
    r.w[24] = v[0]; r.w[25] = v[1];
  }
  const u32x4 sc = *((const u32x4*)(row + 4 * NB * N));
  r.w[28] = sc[0]; r.w[29] = sc[1]; r.w[30] = sc[2]; r.w[31] = sc[3];
}

__device__ inline void load_k_bf16(KRaw& r, const uint8_t* row, int j) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const u32x4 v = *((const u32x4*)(row + (32 * b + 8 * j) * 2));
    r.w[4 * b] = v[0]; r.w[4 * b + 1] = v[1]; r.w[4 * b + 2] = v[2]; r.w[4 * b + 3] = v[3];
  }
}

// QK of block B over a qN_0 row part: the plane MFMAs (query operand of plane p at qb[p * 512 + B * 64 + lane])
// plus the code-bias product, times the block scale d (0 for a lane whose row is not of this kind).
template <int N, int B>
__device__ inline void qk_block(const KRaw& kr, const half8* qb, half8 kbias, float d, floatx4& acc) {
  const int lane = threadIdx.x & 63;
  KPlanes<N> kp;
  dn_piece<N, B>(&kr.w[0], &kr.w[16], &kr.w[24], kp);
  const half8 q0 = qb[B * 64 + lane];
  floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(q0, kbias, floatx4{0, 0, 0, 0}, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(q0, kp.a[0], c, 0, 0, 0);
  if constexpr (Planes<N>::n >= 2) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[512 + B * 64 + lane], kp.a[1], c, 0, 0, 0);
  if constexpr (Planes<N>::n >= 3) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[1024 + B * 64 + lane], kp.a[2], c, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = fmaf(d, c[r], acc[r]);
}

// -2^(N-1) * 2^(q_i - 24) per element: with the plane-0 query operand, minus the code bias 2^(N-1)
template <int N>
__device__ inline half8 k_bias() {
  half8 kb;
#pragma unroll
  for (int i = 0; i < 8; ++i) kb[i] = (_Float16)(-ldexpf(1.0f, N - 1 + dn_bitpos(Planes<N>::w[0], 0, i) - 24));
  return kb;
}

template <int N>
__device__ inline void qk_qrow(const KRaw& kr, const half8* qb, bool use, floatx4& acc) {
  const half8 kb = k_bias<N>();
  float d[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) d[b] = use ? f16f((kr.w[28 + (b >> 1)] >> (16 * (b & 1))) & 0xFFFFu) : 0.0f;
  qk_block<N, 0>(kr, qb, kb, d[0], acc);
  qk_block<N, 1>(kr, qb, kb, d[1], acc);
  qk_block<N, 2>(kr, qb, kb, d[2], acc);
  qk_block<N, 3>(kr, qb, kb, d[3], acc);
  qk_block<N, 4>(kr, qb, kb, d[4], acc);
  qk_block<N, 5>(kr, qb, kb, d[5], acc);
  qk_block<N, 6>(kr, qb, kb, d[6], acc);
  qk_block<N, 7>(kr, qb, kb, d[7], acc);
}

// f16 ring rows: the fp16 values themselves against the shifted fp16 hi / lo query rows.
__device__ inline void qk_f16(const KRaw& kr, const half8* qb, bool use, floatx4& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    u32x4 w = {kr.w[4 * b], kr.w[4 * b + 1], kr.w[4 * b + 2], kr.w[4 * b + 3]};
    if (!use) w = u32x4{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[b * 64 + lane], __builtin_bit_cast(half8, w), acc, 0, 0, 0);
  }
}

__device__ inline void qk_bf16(const KRaw& kr, const bf16x8* qb, bool use, floatx4& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    u32x4 w = {kr.w[4 * b], kr.w[4 * b + 1], kr.w[4 * b + 2], kr.w[4 * b + 3]};
    if (!use) w = u32x4{0u, 0u, 0u, 0u};   // another kind of row: its bytes need not be finite as bf16
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[b * 64 + lane], __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);
  }
}

// ---- V side: channels 4c..4c+3 of one row

struct VRaw {
  uint32_t w[4];   // one word per plane (w <= 3 planes) + the block scale in w[3] (bf16: w[0..1])
};

template <int N>
__device__ inline void load_v_qrow(VRaw& r, const uint8_t* row, int c) {
  constexpr int NB = 8;
  using P = Planes<N>;
  constexpr int w0 = P::w[0], w1 = P::w[1], w2 = P::w[2];
  const int b = c >> 3, j = (c & 7) >> 1;
  const int pc = j * NB + b;
  if constexpr (N == 8) {
    r.w[0] = *((const uint32_t*)(row + pc * 8 + 4 * (c & 1)));
  } else {
    r.w[0] = *((const uint32_t*)(row + 4 * ((pc * w0) / 4)));
    if constexpr (P::n >= 2)
      r.w[1] = *((const uint32_t*)(row + 4 * NB * w0 + 4 * ((pc * w1) / 4)));
    if constexpr (P::n >= 3)
      r.w[2] = *((const uint32_t*)(row + 4 * NB * (w0 + w1) + 4 * ((pc * w2) / 4)));
  }
  r.w[3] = *((const uint16_t*)(row + 4 * NB * N + 2 * b));
}

template <int N>
__device__ inline void v_values(const VRaw& r, int c, float* v) {
  constexpr int NB = 8;
  using P = Planes<N>;
  const int b = c >> 3, j = (c & 7) >> 1, i0 = 4 * (c & 1);
  const int pc = j * NB + b;
  const float d = f16f(r.w[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t u;
    if constexpr (N == 8) {
      u = (r.w[0] >> (8 * k)) & 0xFFu;
    } else {
      u = piece_elem<P::w[0]>(r.w[0], pc, i0 + k);
      if constexpr (P::n >= 2) u |= piece_elem<P::w[1]>(r.w[1], pc, i0 + k) << P::sh[1];
      if constexpr (P::n >= 3) u |= piece_elem<P::w[2]>(r.w[2], pc, i0 + k) << P::sh[2];
    }
    v[k] = (float)((int)u - (1 << (N - 1))) * d;   // exact: integer code times an fp16 scale
  }
}

// ---- one wave step: the sources of 16 list entries and their K and V loads

struct StepRows {
  int pos;                  // this lane's entry (e16), -1 past the range
  bool valid, body;
  uint32_t vmask, bmask;    // entries that are valid / body rows
  KRaw kr;
  VRaw vr[16];
};

// Row sources of one (sequence, KV head): the K and V rows of position (or slot) 0 and the byte stride from one
// position to the next (the rows are position-major: every head's K and V rows of a position sit together).
struct RowSrc {
  const uint8_t *kbody, *vbody, *kring, *vring;
  const int32_t* plist;
  int len, body_len, R, tail, body_stride, ring_stride;
};

__device__ inline void load_pos(StepRows& st, const RowSrc& rs, int g0, int ie) {
  const int idx = g0 + (threadIdx.x & 15);
  int pos = -1;
  if (idx < ie) pos = rs.plist ? rs.plist[idx] : idx;
  st.pos = pos;
}

// (Rows go to local copies first and into st once at the end: stores to st made on some paths only would be
// merged behind a select of their addresses, which keeps st out of registers. Entries with no row keep
// undefined words: their scale is zero (body and q8_0 chains), their bf16 / f16 operand is zeroed, and P.V
// skips them.)
template <int NK, int NV>
__device__ inline void load_rows(StepRows& st, const RowSrc& rs) {
  const int lane = threadIdx.x & 63, j = lane >> 4;
  const int pos = st.pos;
  const bool valid = pos >= 0 && pos < rs.len;
  const bool body = valid && pos < rs.body_len;
  KRaw kr;   // (no zero fill: merging it with the loads would wait for them here)
  if (body) {
    load_k_qrow<NK>(kr, rs.kbody + (size_t)pos * rs.body_stride, j);
  } else if (valid) {
    if (rs.tail == 2) load_k_qrow<8>(kr, rs.kring + (size_t)(pos % rs.R) * rs.ring_stride, j);
    else load_k_bf16(kr, rs.kring + (size_t)(pos % rs.R) * rs.ring_stride, j);
  }
  // V rows of the 16 entries (lane = channel group)
  uint32_t vmask = 0, bmask = 0;
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    const int pt = __builtin_amdgcn_readlane(pos, t);
    VRaw vr;
    if (pt >= 0 && pt < rs.len) {
      vmask |= 1u << t;
      if (pt < rs.body_len) {
        bmask |= 1u << t;
        load_v_qrow<NV>(vr, rs.vbody + (size_t)pt * rs.body_stride, lane);
      } else if (rs.tail == 2) {
        load_v_qrow<8>(vr, rs.vring + (size_t)(pt % rs.R) * rs.ring_stride, lane);
      } else {
        const u32x2 x = *((const u32x2*)(rs.vring + (size_t)(pt % rs.R) * rs.ring_stride + 8 * lane));
        vr.w[0] = x[0];
        vr.w[1] = x[1];
      }
    }
    st.vr[t] = vr;
  }
  st.kr = kr;
  st.valid = valid;
  st.body = body;
  st.vmask = vmask;
  st.bmask = bmask;
}

template <int NK>
__device__ inline void image_k(StepRows& st, const uint8_t* img_k, int app) {
  KRaw im;
  load_k_qrow<NK>(im, img_k, (threadIdx.x & 63) >> 4);
  const bool m = st.pos == app;
#pragma unroll
  for (int k = 0; k < 32; ++k) st.kr.w[k] = m ? im.w[k] : st.kr.w[k];   // selects: no partial writes
}
template <int NV>
__device__ inline void image_v(StepRows& st, const uint8_t* img_v, int app) {
  VRaw im;
  load_v_qrow<NV>(im, img_v, threadIdx.x & 63);
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    const bool m = __builtin_amdgcn_readlane(st.pos, t) == app;
#pragma unroll
    for (int k = 0; k < 4; ++k) st.vr[t].w[k] = m ? im.w[k] : st.vr[t].w[k];
  }
}

// The append of a fused sparse decode step (a cache without a ring): one token of this sequence and KV head
// quantized into body row app_pos, K and V, as the body write of an append does it (thread c owns channel c of
// K and V; a block's 32 values are the 32 lanes of a half-wave). sparse_step_inputs loads the thread's two input
// values (divided by KVarN sigma); sparse_step_emit quantizes them into the zeroed LDS row images img_k / img_v
// (the body row layout), from which the kernel stores them to the body.
__device__ inline void sparse_step_inputs(const GatherArgs& a, const GatherSeq& S, int si, int head, float* x) {
  const Geometry& g = a.g;
  constexpr int D = 256;
  const int c = threadIdx.x & (D - 1);
  const uint8_t* slab = g.arena + S.slab;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* in = kv ? a.v_in : a.k_in;
    x[kv] = bf16_to_f32(in[((size_t)si * g.n_kv_heads + head) * D + c]);
    if (g.kvarn) x[kv] = x[kv] / f16_to_f32(((const uint16_t*)(slab + g.sigma))[((size_t)head * 2 + kv) * D + c]);
  }
}
__device__ inline void sparse_step_emit(const GatherArgs& a, const float* x, uint8_t* img_k, uint8_t* img_v) {
  const Geometry& g = a.g;
  constexpr int D = 256;
  const int c = threadIdx.x & (D - 1);
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const int nb = kv ? g.v_bits : g.k_bits;
    uint16_t dq;
    const uint32_t u = quant_lane(x[kv], nb, &dq);
    uint8_t* row = kv ? img_v : img_k;
    or_code(row, nullptr, true, kv, nb, 0, c, u, D);   // the image was zeroed
    if ((c % kBlock) == 0) ((uint16_t*)(row + 4 * (D / kBlock) * nb))[c / kBlock] = dq;
  }
}

// ---- the kernel

template <int NK, int NV>
__global__ __launch_bounds__(64 * kGWaves) __attribute__((amdgpu_waves_per_eu(kGWaves / 4, kGWaves / 4))) void gather_kernel(GatherArgs a) {
  constexpr int D = 256, G = kPartialHeads, NW = kGWaves;
  __shared__ half8 s_qb[3 * 8 * 64];            // body query operand: [plane][block][lane]
  __shared__ half8 s_qr[8 * 64];                // ring query operand (q8_0: fp16 weighted; bf16: bf16 q)
  __shared__ float s_o[NW][G][D];
  __shared__ float s_ml[NW][2][G];
  __shared__ float s_p[NW][kGroup + 1][G];      // per wave: weights [entry][head], then the step's maxima
  __shared__ float s_amax[NW][2];
  __shared__ __attribute__((aligned(16))) uint8_t s_img[2 * kImgRow];   // fused step: K and V row images

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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = g.ring_slots;
  const int tail = g.tail_dtype;
  const uint8_t* slab = g.arena + S.slab;
  const bool kvarn = g.kvarn != 0;
  const uint16_t* sig = (const uint16_t*)(slab + g.sigma) + (size_t)head * 2 * D;
  const int j = lane >> 4, e16 = lane & 15;
  const int ib = (int)((long)split * S.n_list / S.n_splits);
  const int ie = (int)((long)(split + 1) * S.n_list / S.n_splits);
  const int body_pair = g.row_k + g.row_v, ring_pair = g.ring_row_k + g.ring_row_v;
  const RowSrc rs{slab + g.k_body + rows_k_off(0, head, g.n_kv_heads, body_pair),
                  slab + g.k_body + rows_v_off(0, head, g.n_kv_heads, body_pair, g.row_k),
                  slab + g.k_ring + rows_k_off(0, head, g.n_kv_heads, ring_pair),
                  slab + g.k_ring + rows_v_off(0, head, g.n_kv_heads, ring_pair, g.ring_row_k),
                  a.positions ? a.positions + (size_t)si * a.pos_stride : nullptr,
                  S.len, S.body_len, R, tail, g.n_kv_heads * body_pair, g.n_kv_heads * ring_pair};
  // ---- query operands: wave w builds blocks w + NW k (channels 32 b + 8j + i) for row e16 of the A operand
  constexpr int BPW = 8 / NW;   // blocks per wave
  const int hh = e16 & 7;
  const bool lo_row = e16 >= 8, head_ok = hh < a.group;
  int g0 = ib + kGroup * wave;
  // fused append (a.step): every work-group whose range lists the new position builds its K and V rows in LDS
  // and reads those entries from there; the first split of the KV head writes the rows to global memory at its
  // end (so no work-group waits for another's writes, and none waits for the write)
  const int app = a.step ? S.app_pos : -1;
  bool hit = false;
  float app_x[2] = {0.0f, 0.0f};
  if (app >= 0) {
    sparse_step_inputs(a, S, si, head, app_x);
    for (int idx = ib + tid; idx < ie; idx += 64 * NW) hit |= (rs.plist ? rs.plist[idx] : idx) == app;
    for (int w = tid; w < 2 * kImgRow / 4; w += 64 * NW) ((uint32_t*)s_img)[w] = 0u;
  }

  int e = 0, er = 0;   // exponent shifts of the body and the q8_0 ring operands (the same in every lane)
  {
    float x[BPW][8], xr[BPW][8];
    float am = 0.0f, amr = 0.0f;
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int b = wave + NW * k;
      const u32x4 qw = *(const u32x4*)(a.q + ((size_t)si * a.n_q_heads + head * a.group + (head_ok ? hh : 0)) * D +
                                        32 * b + 8 * j);
      u32x4 sw = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};   // fp16 1.0
      if (kvarn) sw = *(const u32x4*)(sig + 32 * b + 8 * j);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xr[k][i] = head_ok ? bf16f((qw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) : 0.0f;
        x[k][i] = xr[k][i] * f16f((sw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);   // exact in fp32 (8 + 11 bits)
        am = fmaxf(am, fabsf(x[k][i]));
        amr = fmaxf(amr, fabsf(xr[k][i]));
      }
      if (tail == 1) {   // bf16 ring: the query itself in rows 0-7, zero lo rows
        const u32x4 bq = lo_row || !head_ok ? u32x4{0u, 0u, 0u, 0u} : qw;
        ((u32x4*)s_qr)[b * 64 + lane] = bq;
      }
    }
    // one exponent shift per work-group and operand: |q| < 2^9 after it, so that the plane weights (up to
    // 2^6) keep every operand in fp16 range
    am = row16_max(wave_max_16_32(am));
    amr = row16_max(wave_max_16_32(amr));
    if (lane == 0) {
      s_amax[wave][0] = am;
      s_amax[wave][1] = amr;
    }
    if (app >= 0) hit = __syncthreads_or(hit);   // (also publishes s_amax and the zeroed row images)
    else __syncthreads();
    if (app >= 0 && hit) sparse_step_emit(a, app_x, s_img, s_img + kImgRow);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      am = fmaxf(am, s_amax[w][0]);
      amr = fmaxf(amr, s_amax[w][1]);
    }
    e = am > 0.0f ? ilogbf(am) - 8 : 0;
    er = amr > 0.0f ? ilogbf(amr) - 8 : 0;
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int b = wave + NW * k;
      float part[8], partr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xs = ldexpf(x[k][i], -e);
        const _Float16 h = (_Float16)xs;
        part[i] = lo_row ? (float)(_Float16)(xs - (float)h) : (float)h;
        const float xq = ldexpf(xr[k][i], -er);
        const _Float16 hq = (_Float16)xq;
        partr[i] = lo_row ? (float)(_Float16)(xq - (float)hq) : (float)hq;
      }
#pragma unroll
      for (int p = 0; p < Planes<NK>::n; ++p) {
        const int w = Planes<NK>::w[p];
        const int slot = w == 8 ? 0 : b % (4 / w);
        half8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)ldexpf(part[i], Planes<NK>::sh[p] - dn_bitpos(w, slot, i));   // exact
        s_qb[p * 512 + b * 64 + lane] = v;
      }
      if (tail == 2 || tail == 3) {   // q8_0 or f16 ring: the shifted query as fp16 hi / lo rows
        half8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)partr[i];   // 8-bit plane: every field at bit 0
        s_qr[b * 64 + lane] = v;
      }
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
  const float qsc = a.scale * kLog2e;
  const float qmul_b = qsc * ldexpf(1.0f, e + 24);   // body scores: C * d * 2^(e + 24)
  const float qmul_r = tail == 2 ? qsc * ldexpf(1.0f, er + 24) : tail == 3 ? qsc * ldexpf(1.0f, er) : qsc;

  float (*sp)[G] = s_p[wave];

  float m[G], o[G][4], m4[4], l4[4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[h][k] = 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {   // the running maximum and sum of heads 4 (j & 1) + r (sum: lanes 0-31)
    m4[r] = kNegBig;
    l4[r] = 0.0f;
  }

  for (; g0 < ie; g0 += kGroup * NW) {
    StepRows st;
    load_pos(st, rs, g0, ie);
    load_rows<NK, NV>(st, rs);
    if (hit) image_k<NK>(st, s_img, app);
    const uint32_t vmask = st.vmask, bmask = st.bmask;
    const bool valid = st.valid, body = st.body, ring = valid && !body;
    const KRaw& kr = st.kr;
    if (!vmask) continue;
    // ---- scores: lane (j, e16) ends with rows 4j..4j+3 of the 16 x 16 product (query rows x entries)
    floatx4 accb = {0, 0, 0, 0}, accr = {0, 0, 0, 0};
    if (bmask) qk_qrow<NK>(kr, s_qb, body, accb);
    if (vmask & ~bmask) {
      if (tail == 2) qk_qrow<8>(kr, s_qr, ring, accr);
      else if (tail == 3) qk_f16(kr, s_qr, ring, accr);
      else qk_bf16(kr, (const bf16x8*)s_qr, ring, accr);
    }
    if (hit) image_v<NV>(st, s_img + kImgRow, app);   // after QK: the V loads had that long to arrive
    float s[4], mx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = sum_xor32(accb[r] * qmul_b + accr[r] * qmul_r);   // hi rows + lo rows: heads 4 (j & 1) + r
      s[r] = valid ? s[r] : -INFINITY;
      mx[r] = row16_max(s[r]);
    }
    // ---- online softmax: the step's maxima of all 8 heads to every lane through LDS
    if (lane == 0 || lane == 16) *(floatx4*)&sp[kGroup][4 * j] = floatx4{mx[0], mx[1], mx[2], mx[3]};
    __builtin_amdgcn_wave_barrier();
    const floatx4 mlo = *(const floatx4*)&sp[kGroup][0], mhi = *(const floatx4*)&sp[kGroup][4];
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mn = fmaxf(m[h], h < 4 ? mlo[h] : mhi[h - 4]);
      alpha[h] = __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
    }
    {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {   // the same maxima as m[4 (j & 1) + r], from this lane's own row
        const float mn = fmaxf(m4[r], mx[r]);
        p[r] = __builtin_amdgcn_exp2f(s[r] - mn);
        l4[r] = l4[r] * __builtin_amdgcn_exp2f(m4[r] - mn) + p[r];
        m4[r] = mn;
      }
      if (lane < 32) *(floatx4*)&sp[e16][4 * j] = floatx4{p[0], p[1], p[2], p[3]};
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) o[h][k] *= alpha[h];
    __builtin_amdgcn_wave_barrier();
    // ---- P.V for the 16 entries (a step of body rows only is straight-line code: the weight reads of the
    // next entries can be issued ahead of the arithmetic)
    auto pv = [&](int t, const float* v) {
      const floatx4 p0 = *(const floatx4*)&sp[t][0], p1 = *(const floatx4*)&sp[t][4];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = h < 4 ? p0[h] : p1[h - 4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[h][k] = fmaf(ph, v[k], o[h][k]);
      }
    };
    if (bmask == 0xFFFFu) {
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        float v[4];
        v_values<NV>(st.vr[t], lane, v);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] *= sv[k];
        pv(t, v);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        if (!(vmask & (1u << t))) continue;
        float v[4];
        const VRaw& vr = st.vr[t];
        if (bmask & (1u << t)) {
          v_values<NV>(vr, lane, v);
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] *= sv[k];
        } else if (tail == 2) {
          v_values<8>(vr, lane, v);
        } else if (tail == 3) {
          v[0] = f16f(vr.w[0] & 0xFFFFu);
          v[1] = f16f(vr.w[0] >> 16);
          v[2] = f16f(vr.w[1] & 0xFFFFu);
          v[3] = f16f(vr.w[1] >> 16);
        } else {
          v[0] = bf16f(vr.w[0] & 0xFFFFu);
          v[1] = bf16f(vr.w[0] >> 16);
          v[2] = bf16f(vr.w[1] & 0xFFFFu);
          v[3] = bf16f(vr.w[1] >> 16);
        }
        pv(t, v);
      }
    }
    __builtin_amdgcn_wave_barrier();   // the next step's writes of sp come after these reads
  }

  // ---- wave partials to LDS, then the work-group merge
  float lsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lsum[r] = row16_sum(lane < 32 ? l4[r] : 0.0f);
  if (lane == 0 || lane == 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_ml[wave][1][4 * j + r] = lsum[r];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) s_ml[wave][0][h] = m[h];
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k) s_o[wave][h][4 * lane + k] = o[h][k];
  __syncthreads();
  float* part = a.partials + (((size_t)si * g.n_kv_heads + head) * a.max_splits + split) * (G * (D + 2));
  const int c = tid % D;
#pragma unroll
  for (int h = tid / D; h < G; h += 64 * NW / D) {
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0][h]);
    float O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) O += s_o[w][h][c] * __builtin_amdgcn_exp2f(s_ml[w][0][h] - M);
    part[2 * G + h * D + c] = O;
  }
  if (tid < G) {
    float M = kNegBig, L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0][tid]);
#pragma unroll
    for (int w = 0; w < NW; ++w) L += s_ml[w][1][tid] * __builtin_amdgcn_exp2f(s_ml[w][0][tid] - M);
    part[tid] = M;
    part[G + tid] = L;
  }
  // the new position's rows in global memory, once per KV head (no work-group of this launch reads them from
  // there: those that list the position read the LDS image), after the split's own work: the rows are built in
  // the LDS images (already there if this work-group lists the position) and stored with 16-byte writes
  if (app >= 0 && split == 0) {
    if (!hit) sparse_step_emit(a, app_x, s_img, s_img + kImgRow);
    __syncthreads();
    const int body_pair = g.row_k + g.row_v, nk16 = g.row_k / 16, nv16 = g.row_v / 16;
    uint8_t* rows = g.arena + S.slab + g.k_body;
    if (tid < nk16)
      ((u32x4*)(rows + rows_k_off(app, head, g.n_kv_heads, body_pair)))[tid] = ((const u32x4*)s_img)[tid];
    else if (tid < nk16 + nv16)
      ((u32x4*)(rows + rows_v_off(app, head, g.n_kv_heads, body_pair, g.row_k)))[tid - nk16] =
          ((const u32x4*)(s_img + kImgRow))[tid - nk16];
  }
}

template <int NK, int NV>
hipError_t launch_gather_t(const GatherArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(gather_kernel<NK, NV>, dim3(grid_x), dim3(64 * kGWaves), s, e0, e1, a);
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
