// The library's static scratch buffer: device memory for the split partials of kvq_decode_attn_noalloc, the
// decode entry point for callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Every GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device address, per device, comes from
// hipGetSymbolAddress, called once per device with that device current, and only that address is ever
// passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_kernels.h"

static __device__ __align__(256) uint8_t scratch[kvq::kScratchBytes];

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_device_ptr(int device, void** out) {
  if (!out || device < 0 || device >= kMaxDevices) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return hipSuccess;
}

}  // namespace kvq
