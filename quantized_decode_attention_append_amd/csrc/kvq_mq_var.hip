// Multi-query kernel instantiations that read qN_1 bodies (a scale and a minimum per block) and token-axis K
// (KIVI-style per-channel K blocks); built apart from kvq_mq.hip so that the two sets compile in parallel.
#include "kvq_mq_impl.h"

namespace kvq {

hipError_t launch_mq_variant(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_mq_dispatch<true>(a, grid_x, s, e0, e1);
}

}  // namespace kvq
