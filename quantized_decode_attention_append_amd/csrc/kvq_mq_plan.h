// Query-block size of the multi-query launches, shared by the host plan and the kernel dispatch.
#pragma once

#include "kvq_kernels.h"

namespace kvq {

// Queries per multi-query block. Without qN_1 bodies and token-axis K a wave computes two queries (their heads
// in the 16 columns of one fp16 query operand): a block holds 16, or 8 for a KVarN cache (its K remainders take
// the LDS of the raw staging that larger blocks need). With them a wave computes one query (its operand a hi / lo
// pair of fp16 columns per head) and a block holds 8.
constexpr int kMqBlockPair = 16, kMqBlockSingle = 8;

inline bool mq_pairs(const Geometry& g) { return !(g.k_min || g.v_min || g.k_axis); }
inline int mq_block_queries(const Geometry& g) { return mq_pairs(g) && !g.kvarn ? kMqBlockPair : kMqBlockSingle; }

hipError_t launch_mq_pair(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_mq_pair_kv(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1);

}  // namespace kvq
