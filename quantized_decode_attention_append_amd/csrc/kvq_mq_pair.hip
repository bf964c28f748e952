// Launches of the two-queries-per-wave multi-query kernel (kvq_mq_pair_impl.h) for caches without KVarN; the
// KVarN instantiations are built in kvq_mq_pair_kv.hip.
#include "kvq_mq_pair_impl.h"

namespace kvq {

hipError_t launch_mq_pair(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.g.kvarn) return launch_mq_pair_kv(a, grid_x, s, e0, e1);
  return launch_pair_dispatch<false>(a, grid_x, s, e0, e1);
}

}  // namespace kvq
