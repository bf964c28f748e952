// Query-block size of the multi-query launches, shared by the host plan and the kernel dispatch.
#pragma once

#include "kvq_kernels.h"

namespace kvq {

// Queries per multi-query block. Where the query operand is one fp16 column per head (no KVarN, no qN_1 body, no
// token-axis K) a wave computes two queries and a block holds 16; otherwise a wave computes one query (its
// operand a hi / lo pair of fp16 columns per head) and a block holds 8.
constexpr int kMqBlockPair = 16, kMqBlockSingle = 8;

inline bool mq_pairs(const Geometry& g) { return !(g.kvarn || g.k_min || g.v_min || g.k_axis); }
inline int mq_block_queries(const Geometry& g) { return mq_pairs(g) ? kMqBlockPair : kMqBlockSingle; }

hipError_t launch_mq_pair(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0, hipEvent_t e1);

}  // namespace kvq
