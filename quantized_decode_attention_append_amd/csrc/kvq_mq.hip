// Multi-query kernel launches: caches with qN_1 bodies or token-axis K run the one-query-per-wave kernel of
// kvq_mq_impl.h (instantiations built in kvq_mq_var.hip), every other cache the two-queries-per-wave kernel
// (kvq_mq_pair.hip, kvq_mq_pair_kv.hip); and the split merge.
#include "kvq_mq_impl.h"
#include "kvq_mq_plan.h"

namespace kvq {

hipError_t launch_mq_variant(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1);

hipError_t launch_mq(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (!mq_pairs(a.g)) return launch_mq_variant(a, grid_x, s, e0, e1);
  return launch_mq_pair(a, grid_x, s, e0, e1);
}

hipError_t launch_mq_combine(const MqArgs& a, int rows, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_k(mq_combine_kernel, dim3(rows * a.g.n_kv_heads, a.group), dim3(1024), s, e0, e1, a);
}

}  // namespace kvq
