// Launches of the two-queries-per-wave multi-query kernel (kvq_mq_pair_impl.h) for KVarN caches.
#include "kvq_mq_pair_impl.h"

namespace kvq {

hipError_t launch_mq_pair_kv(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_pair_dispatch<true>(a, grid_x, s, e0, e1);
}

}  // namespace kvq
