// Streaming-read probe: the HBM read rate this GPU sustains for a plain read-only pass over a buffer, measured
// beside the decode kernels (whose traffic is ~96 % reads). Not part of the cache's C ABI: built into its own
// library (libkvq_probe.so) and called only by the benchmark.
//
// Every thread reads `unroll` 16-byte vectors per trip, strided by the grid so that each load instruction of a
// wave covers 1 KiB contiguous, XORs them into a register and writes one word per work-group at the end (so no
// load can be removed). Loads are ordinary or nontemporal (the decode kernels stream their tiles with
// nontemporal loads).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(1024) void read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= NT ? __builtin_nontemporal_load(p + i) : p[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t s[16];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) y ^= s[w];
    sink[blockIdx.x] = y;
  }
}

template <int U, bool NT>
hipError_t launch(const void* src, size_t n16, void* sink, int grid, int block, hipStream_t s) {
  hipLaunchKernelGGL((read_kernel<U, NT>), dim3(grid), dim3(block), 0, s, (const u32x4*)src, n16, (uint32_t*)sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from device memory `src` once. sink: device memory of at
// least `grid` 32-bit words. grid >= 1 work-groups of `block` threads (64..1024, a multiple of 64); unroll: 1, 2,
// 4 or 8 vectors in flight per thread; nontemporal: 0 or 1. Returns a hipError_t (0 = launched).
int kvq_probe_read(const void* src, size_t bytes, void* sink, int grid, int block, int unroll, int nontemporal,
                   void* stream) {
  if (!src || !sink || bytes % 16 || ((uintptr_t)src) % 16 || grid < 1 || block < 64 || block > 1024 || block % 64)
    return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const hipStream_t s = (hipStream_t)stream;
#define KVQ_PROBE(U)                                                                                  \
  if (unroll == U)                                                                                    \
    return (int)(nontemporal ? launch<U, true>(src, n16, sink, grid, block, s)                        \
                             : launch<U, false>(src, n16, sink, grid, block, s));
  KVQ_PROBE(1) KVQ_PROBE(2) KVQ_PROBE(4) KVQ_PROBE(8)
#undef KVQ_PROBE
  return (int)hipErrorInvalidValue;
}

}  // extern "C"
