// Append-side kernels: KVarN calibration, qN_0 quantization into the body (also used for the q8_0 ring
// and for requantizing ring rows that leave the window), and the bf16 tail-ring write.
//
// Arithmetic follows the symmetric qN_0 block format of the BeeLlama page (32 values, one fp16 scale, no
// offset): d = amax / qmax in IEEE fp32, fp16 round-to-nearest-even saturating at 65504, codes
// rne(x / d16) clamped to [-qmax, qmax], stored biased by 2^(N-1). This file is built with
// -ffp-contract=off and correctly rounded fp32 division, so the codes are bit-identical to a plain
// IEEE evaluation.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kvq_kernels.h"

namespace kvq {
namespace {

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ inline float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Quantize 32 fp32 values to N-bit biased codes and an fp16 scale (bit pattern).
__device__ inline void quant_block(const float* x, int n_bits, uint8_t* u, uint16_t* d16_bits) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float qmax = (float)((1 << (n_bits - 1)) - 1);
  float d = amax / qmax;                       // correctly rounded (see build flags)
  d = fminf(d, 65504.0f);
  _Float16 h = (_Float16)d;                     // RNE
  float dh = (float)h;
  const int off = 1 << (n_bits - 1);
  if (dh == 0.0f) {
#pragma unroll
    for (int i = 0; i < 32; ++i) u[i] = (uint8_t)off;
    *d16_bits = 0;
    return;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float c = rintf(x[i] / dh);                  // round half to even
    c = fminf(fmaxf(c, -qmax), qmax);
    u[i] = (uint8_t)((int)c + off);
  }
  *d16_bits = __builtin_bit_cast(uint16_t, h);
}

// fp32 value of a q8_0 round trip of 32 values (the 8-bit ring representation).
__device__ inline void q8_round_trip(float* x) {
  uint8_t u[32];
  uint16_t d;
  quant_block(x, 8, u, &d);
  float dh = f16_to_f32(d);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = (float)((int)u[i] - 128) * dh;   // exact product
}

// fp64 -> fp16 bits for a KVarN scale: RNE, 0 / non-finite -> 1, clamped to [2^-14, 65504].
__device__ inline uint16_t sigma_to_f16(double s) {
  if (!(s > 0.0) || !isfinite(s)) return 0x3C00;
  if (s >= 65504.0) return 0x7BFF;
  if (s < 6.103515625e-05) return 0x0400;
  int e;
  double m = frexp(s, &e);                    // s = m * 2^e, m in [0.5, 1)
  double r = rint(ldexp(m, 11));              // 11 significant bits, RNE (exact in fp64)
  double v = ldexp(r, e - 11);                // exactly representable in fp16 (normal range)
  if (v > 65504.0) v = 65504.0;
  _Float16 h = (_Float16)(float)v;            // exact conversions
  return __builtin_bit_cast(uint16_t, h);
}

// ------------------------------------------------------------------------------ calibration

__global__ __launch_bounds__(256) void calibrate_kernel(CalibArgs a) {
  const CalibItem& it = a.items[blockIdx.x];
  const int head = blockIdx.y;
  const int kv = blockIdx.z;
  const Geometry& g = a.g;
  const int D = g.head_dim;
  const uint16_t* in = kv ? a.v_in : a.k_in;
  uint16_t* sig = (uint16_t*)(g.arena + it.slab + g.sigma) + ((size_t)head * 2 + kv) * D;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    double acc = 0.0;
    for (int t = 0; t < it.n; ++t) {
      double x = (double)bf16_to_f32(in[((size_t)(it.src_row + t) * g.n_kv_heads + head) * D + c]);
      acc += x * x;                            // each square is exact in fp64
    }
    double ms = acc / (double)it.n;
    sig[c] = sigma_to_f16(sqrt(ms));
  }
}

// ------------------------------------------------------------------------------ body write

// Source values (fp32) of one (position, block) for K or V.
struct SrcCtx {
  const Geometry* g;
  const uint8_t* slab;
  const uint16_t* in;    // input for this tensor (K or V)
  int kv;                // 0 K, 1 V
  int head;
};

// Read 32 consecutive channels [32b, 32b+32) of position p from the ring (fp32 ring representation).
__device__ inline void load_ring_block(const SrcCtx& s, int p, int b, float* x) {
  const Geometry& g = *s.g;
  const int D = g.head_dim;
  const int NB = D / kBlock;
  const int R = g.ring_slots;
  const int slot = p % R;
  if (g.tail_dtype == 1) {
    if (s.kv == 0) {
      const uint16_t* row = (const uint16_t*)(s.slab + g.k_ring) + ((size_t)s.head * R + slot) * D + 32 * b;
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(row[i]);
    } else {
      const uint8_t* tile = s.slab + g.v_ring + ((size_t)s.head * (R / kTile) + slot / kTile) * g.ring_tile_v;
      const int t = slot % kTile;
      const int j = (t % 16) / 4;
      const int e = (t % 4) + 4 * (t / 16);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int c = 32 * b + i;
        const int lane = 16 * j + (c % 16);
        const uint16_t* p16 = (const uint16_t*)(tile + (size_t)(c / 16) * 64 * 16 + lane * 16) + e;
        x[i] = bf16_to_f32(*p16);
      }
    }
    return;
  }
  // q8_0 ring
  if (s.kv == 0) {
    const uint8_t* row = s.slab + g.k_ring + ((size_t)s.head * R + slot) * g.ring_row_k;
    const float dh = f16_to_f32(((const uint16_t*)(row + NB * 32))[b]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[8 * j + i] = (float)((int)row[(j * NB + b) * 8 + i] - 128) * dh;
  } else {
    const uint8_t* tile = s.slab + g.v_ring + ((size_t)s.head * (R / kTile) + slot / kTile) * g.ring_tile_v;
    const int t = slot % kTile;
    const int j = (t % 16) / 4;
    const int e = (t % 4) + 4 * (t / 16);
    const int NT = D / 16;
    const float dh = f16_to_f32(((const uint16_t*)(tile + 32 * D))[t * NB + b]);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int c = 32 * b + i;
      const int lane = 16 * j + (c % 16);
      const uint8_t code = tile[vtile_lane_byte(lane, (c / 16) * 8 + e, NT, 8)];
      x[i] = (float)((int)code - 128) * dh;
    }
  }
}

__device__ inline void load_input_block(const SrcCtx& s, int row, int b, float* x) {
  const Geometry& g = *s.g;
  const uint16_t* src = s.in + ((size_t)row * g.n_kv_heads + s.head) * g.head_dim + 32 * b;
  const uint4* v = (const uint4*)src;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 w = v[q];
    uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[8 * q + 2 * k] = __uint_as_float(ww[k] << 16);
      x[8 * q + 2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
    }
  }
}

// Bits of one plane of a piece: element i of piece slot p at 16*(i&1) + 4*w*p + w*(i>>1).
__device__ inline uint32_t piece_bits(const uint8_t* u8codes, int w, int shift, int slot) {
  uint32_t bits = 0;
  const uint32_t m = (1u << w) - 1;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    bits |= ((u8codes[i] >> shift) & m) << (16 * (i & 1) + 4 * w * slot + w * (i >> 1));
  return bits;
}

__global__ __launch_bounds__(256) void body_write_kernel(WriteArgs a) {
  __shared__ uint8_t vcodes[kTile][256];
  const Geometry& g = a.g;
  const int wg = blockIdx.x;
  const int head = blockIdx.y;
  int it = 0;
  while (it + 1 < a.n_items && a.items[it + 1].wg_begin <= wg) ++it;
  const WriteItem& w = a.items[it];
  const int tile = w.tile0 + (wg - w.wg_begin);
  const int D = g.head_dim;
  const int NB = D / kBlock;
  const int NT = D / 16;
  const int NK = a.dst_ring ? 8 : g.k_bits;
  const int NV = a.dst_ring ? 8 : g.v_bits;
  const int R = g.ring_slots;
  uint8_t* slab = g.arena + w.slab;

  int row_k;
  uint8_t* kbase;
  uint8_t* vtile;
  int vtile_bytes;
  if (a.dst_ring) {
    row_k = g.ring_row_k;
    kbase = slab + g.k_ring + (size_t)head * R * row_k;
    vtile_bytes = g.ring_tile_v;
    vtile = slab + g.v_ring + ((size_t)head * (R / kTile) + ((tile * kTile) % R) / kTile) * vtile_bytes;
  } else {
    row_k = g.row_k;
    kbase = slab + g.k_body + (size_t)head * g.cap32 * row_k;
    vtile_bytes = g.tile_v;
    vtile = slab + g.v_body + ((size_t)head * (g.cap32 / kTile) + tile) * vtile_bytes;
  }
  const int vcode_bytes = 4 * D * NV;   // 32 positions * D * NV / 8

  SrcCtx sk{&g, slab, a.k_in, 0, head};
  SrcCtx sv{&g, slab, a.v_in, 1, head};

  // ---- phase 1: thread (t, b) quantizes block b of position t for K and V
  const int tid = threadIdx.x;
  const int t = tid / NB;
  const int b = tid % NB;
  const int p = tile * kTile + t;
  const bool active = (t < kTile) && p >= w.p0 && p < w.p1;
  float xk[32], xv[32];
  if (active) {
    if (p >= w.len_old) {
      const int row = w.src_row + (p - w.len_old);
      load_input_block(sk, row, b, xk);
      load_input_block(sv, row, b, xv);
      if (!a.dst_ring && g.tail_dtype == 2 && R > 0) {   // through the q8_0 ring representation
        q8_round_trip(xk);
        q8_round_trip(xv);
      }
    } else {
      load_ring_block(sk, p, b, xk);
      load_ring_block(sv, p, b, xv);
    }
    if (!a.dst_ring && g.kvarn) {
      const uint16_t* sig = (const uint16_t*)(slab + g.sigma) + (size_t)head * 2 * D;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        xk[i] = xk[i] / f16_to_f32(sig[32 * b + i]);
        xv[i] = xv[i] / f16_to_f32(sig[D + 32 * b + i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) xk[i] = xv[i] = 0.0f;
  }
  uint8_t uk[32], uv[32];
  uint16_t dk, dv;
  quant_block(xk, NK, uk, &dk);
  quant_block(xv, NV, uv, &dv);

  // K row: planes of pieces (j, b); words shared by neighbouring blocks are merged with shuffles.
  uint8_t* krow = kbase + (size_t)(a.dst_ring ? (p % (R > 0 ? R : 1)) : p) * row_k;
  int plane_off = 0;
  for (int pl = 0; pl < plane_count(NK); ++pl) {
    const int wdt = plane_width(NK, pl);
    const int sh = plane_shift(NK, pl);
    for (int j = 0; j < 4; ++j) {
      const uint8_t* cj = uk + 8 * j;
      if (wdt == 8) {
        if (active) {
          uint32_t lo = cj[0] | (cj[1] << 8) | (cj[2] << 16) | ((uint32_t)cj[3] << 24);
          uint32_t hi = cj[4] | (cj[5] << 8) | (cj[6] << 16) | ((uint32_t)cj[7] << 24);
          *(uint2*)(krow + plane_off + (j * NB + b) * 8) = make_uint2(lo, hi);
        }
      } else {
        const int per = 4 / wdt;
        uint32_t bits = piece_bits(cj, wdt, sh, b % per);
        if (per >= 2) bits |= __shfl_xor(bits, 1);
        if (per >= 4) bits |= __shfl_xor(bits, 2);
        if (active && (b % per) == 0)
          *(uint32_t*)(krow + plane_off + j * NB * wdt + (b / per) * 4) = bits;
      }
    }
    plane_off += 4 * NB * wdt;
  }
  if (active) {
    ((uint16_t*)(krow + NB * 4 * NK))[b] = dk;
    ((uint16_t*)(vtile + vcode_bytes))[t * NB + b] = dv;
  }
  if (t < kTile) {
#pragma unroll
    for (int i = 0; i < 32; ++i) vcodes[t][32 * b + i] = uv[i];
  }
  __syncthreads();

  // ---- phase 2: V tile pieces, read-modify-write of the words this call touches
  const int lane = tid & 63;
  const int q = tid >> 6;
  const int d16 = lane & 15;
  const int j = lane >> 4;
  uint32_t inmask = 0;   // bit e set when element e's tile position is written by this call
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pp = tile * kTile + tile_pos(j, e);
    if (pp >= w.p0 && pp < w.p1) inmask |= 1u << e;
  }
  if (inmask == 0) return;
  int vplane_off = 0;
  for (int pl = 0; pl < plane_count(NV); ++pl) {
    const int wdt = plane_width(NV, pl);
    const int sh = plane_shift(NV, pl);
    const uint32_t m = (1u << wdt) - 1;
    const int run_dwords = NT * wdt / 4;
    for (int k = q; k < run_dwords; k += 4) {
      uint32_t bits = 0, mask = 0;
      if (wdt == 8) {
        const int n = k / 2;
        const int c = 16 * n + d16;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int e = 4 * (k & 1) + bb;
          if (inmask & (1u << e)) {
            bits |= (uint32_t)vcodes[tile_pos(j, e)][c] << (8 * bb);
            mask |= 0xFFu << (8 * bb);
          }
        }
      } else {
        const int per = 4 / wdt;
        for (int s = 0; s < per; ++s) {
          const int n = k * per + s;
          const int c = 16 * n + d16;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (inmask & (1u << e)) {
              const int pos = 16 * (e & 1) + 4 * wdt * s + wdt * (e >> 1);
              bits |= ((uint32_t)(vcodes[tile_pos(j, e)][c] >> sh) & m) << pos;
              mask |= m << pos;
            }
          }
        }
      }
      uint32_t* dst = (uint32_t*)(vtile + vplane_off + vtile_lane_byte(lane, 4 * k, NT, wdt));
      if (mask == 0xFFFFFFFFu) {
        *dst = bits;
      } else if (mask) {
        *dst = (*dst & ~mask) | bits;
      }
    }
    vplane_off += 64 * NT * wdt;
  }
}

// ------------------------------------------------------------------------------ bf16 ring write

__global__ __launch_bounds__(256) void bf16_ring_write_kernel(WriteArgs a) {
  const Geometry& g = a.g;
  const int wg = blockIdx.x;
  const int head = blockIdx.y;
  int it = 0;
  while (it + 1 < a.n_items && a.items[it + 1].wg_begin <= wg) ++it;
  const WriteItem& w = a.items[it];
  const int tile = w.tile0 + (wg - w.wg_begin);
  const int D = g.head_dim;
  const int NB = D / kBlock;
  const int R = g.ring_slots;
  uint8_t* slab = g.arena + w.slab;
  const int tid = threadIdx.x;
  const int t = tid / NB;
  const int b = tid % NB;
  const int p = tile * kTile + t;
  if (t >= kTile || p < w.p0 || p >= w.p1) return;
  const int row = w.src_row + (p - w.len_old);
  const int slot = p % R;
  const uint16_t* ks = a.k_in + ((size_t)row * g.n_kv_heads + head) * D + 32 * b;
  const uint16_t* vs = a.v_in + ((size_t)row * g.n_kv_heads + head) * D + 32 * b;
  uint16_t* kd = (uint16_t*)(slab + g.k_ring) + ((size_t)head * R + slot) * D + 32 * b;
#pragma unroll
  for (int q = 0; q < 4; ++q) ((uint4*)kd)[q] = ((const uint4*)ks)[q];
  uint8_t* vt = slab + g.v_ring + ((size_t)head * (R / kTile) + slot / kTile) * g.ring_tile_v;
  const int ts = slot % kTile;
  const int j = (ts % 16) / 4;
  const int e = (ts % 4) + 4 * (ts / 16);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int c = 32 * b + i;
    const int lane = 16 * j + (c % 16);
    ((uint16_t*)(vt + (size_t)(c / 16) * 64 * 16 + lane * 16))[e] = vs[i];
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs& a, int n_items, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(n_items, a.g.n_kv_heads, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_body_write(const WriteArgs& a, int n_wgs, hipStream_t s) {
  hipLaunchKernelGGL(body_write_kernel, dim3(n_wgs, a.g.n_kv_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bf16_ring_write(const WriteArgs& a, int n_wgs, hipStream_t s) {
  hipLaunchKernelGGL(bf16_ring_write_kernel, dim3(n_wgs, a.g.n_kv_heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace kvq
