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
#include "kvq_write.h"

namespace kvq {
namespace {


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

__global__ __launch_bounds__(512) void body_write_kernel(WriteArgs a) {
  __shared__ WriteCodes codes;
  body_write_wg(a, blockIdx.x, blockIdx.y, codes);
}

__global__ __launch_bounds__(512) void bf16_ring_write_kernel(WriteArgs a) {
  bf16_ring_write_wg(a, blockIdx.x, blockIdx.y);
}

// A decode step's append and evict in one launch: work-groups [0, ring_wgs) write the new tokens into the
// ring, the rest requantize ring rows that were already there into the body. The two touch disjoint bytes
// (the host only fuses calls whose evicted positions precede the appended ones and fit the ring together).
__global__ __launch_bounds__(512) void step_write_kernel(StepArgs a) {
  __shared__ WriteCodes codes;
  const int x = blockIdx.x;
  if (x < a.ring_wgs) {
    if (a.ring.g.tail_dtype != 2) bf16_ring_write_wg(a.ring, x, blockIdx.y);   // bf16 or f16 values
    else body_write_wg(a.ring, x, blockIdx.y, codes);
  } else {
    body_write_wg(a.body, x - a.ring_wgs, blockIdx.y, codes);
  }
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs& a, int n_items, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(calibrate_kernel, dim3(n_items, a.g.n_kv_heads, 2), dim3(256), s, e0, e1, a);
}

hipError_t launch_body_write(const WriteArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(body_write_kernel, dim3(n_wgs, a.g.n_kv_heads), dim3(512), s, e0, e1, a);
}

hipError_t launch_bf16_ring_write(const WriteArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(bf16_ring_write_kernel, dim3(n_wgs, a.g.n_kv_heads), dim3(512), s, e0, e1, a);
}

hipError_t launch_step_write(const StepArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(step_write_kernel, dim3(n_wgs, a.ring.g.n_kv_heads), dim3(512), s, e0, e1, a);
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
