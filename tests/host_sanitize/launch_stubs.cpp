// Stand-ins for the kernel launchers of the kvq library, for a host-only build of kvq_host.cpp: each checks the
// launch shape it is given and returns success without touching device memory, so every host path of the C ABI
// (validation, planning, workspace checks, error returns) runs on a machine without a GPU.
#include <cstdio>
#include <cstdlib>

#include "kvq_kernels.h"

namespace {
long g_launches = 0;
void check_grid(const char* what, long grid, int n_seqs) {
  ++g_launches;
  if (grid <= 0 || grid > (1L << 24) || n_seqs < 0 || n_seqs > kvq::kMaxBatch) {
    std::fprintf(stderr, "launch stub: %s with grid %ld, %d sequences\n", what, grid, n_seqs);
    std::abort();
  }
}
}  // namespace

extern "C" long kvq_stub_launches() { return g_launches; }

namespace kvq {
hipError_t launch_calibrate(const CalibArgs& a, int n_items, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("calibrate", n_items, 0);
  return hipSuccess;
}
hipError_t launch_body_write(const WriteArgs& a, int n_wgs, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("body_write", n_wgs, a.n_items);
  return hipSuccess;
}
hipError_t launch_bf16_ring_write(const WriteArgs& a, int n_wgs, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("ring_write", n_wgs, a.n_items);
  return hipSuccess;
}
hipError_t launch_step_write(const StepArgs& a, int n_wgs, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("step_write", n_wgs, 0);
  return hipSuccess;
}
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t) {
  check_grid("fill_zero", p ? 1 : 0, 0);
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, int grid_x, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("decode", grid_x, a.n_seqs);
  return hipSuccess;
}
hipError_t launch_gather(const GatherArgs& a, int grid_x, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("gather", grid_x, a.n_seqs);
  return hipSuccess;
}
hipError_t launch_combine(const CombineArgs& a, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("combine", (long)a.n_seqs * a.n_kv_heads, a.n_seqs);
  return hipSuccess;
}
hipError_t launch_index_write(const IndexWriteArgs& a, int n_positions, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("index_write", n_positions, 0);
  return hipSuccess;
}
hipError_t launch_mq(const MqArgs& a, int grid_x, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("mq", grid_x, 0);
  return hipSuccess;
}
hipError_t launch_mq_combine(const MqArgs& a, int rows, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("mq_combine", rows, 0);
  return hipSuccess;
}
hipError_t launch_index_select(const IndexArgs& a, int total_wgs, hipStream_t, hipEvent_t, hipEvent_t) {
  check_grid("index_select", total_wgs, 0);
  return hipSuccess;
}
hipError_t scratch_device_ptr(int, void** ptr) {
  *ptr = (void*)(uintptr_t)0x7f0000000000ull;
  return hipSuccess;
}
}  // namespace kvq
