// Kernel argument blocks and launch wrappers shared by the kvq host code and its kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq_format.h"

namespace kvq {

constexpr int kMaxBatch = 64;      // sequences per call (kernel arguments are passed by value)
constexpr int kPartialHeads = 8;   // query heads per KV head handled by one decode work-group
constexpr int kMaxSplits = 1024;   // split partials per (sequence, KV head)

// Geometry of one (layer) of the arena, as the kernels need it.
struct Geometry {
  uint8_t* arena;
  size_t slab_bytes;
  size_t k_body, v_body, k_ring, v_ring, sigma, index;   // region offsets within a slab
  int cap32, row_k, row_v, tile_k, tile_v, ring_row_k, ring_row_v, ring_tile_k, ring_tile_v, ring_slots;
  int n_kv_heads, head_dim, k_bits, v_bits, kvarn, tail_dtype;
  int layout;                                      // 0: V tiles, 1: V rows
  int k_min, v_min;                                // qN_1 K / V body (scale and minimum per block)
  int k_axis;                                      // 1: token-axis K (a block = 32 positions of one channel)
};

// ---------------------------------------------------------------- append side

// KVarN calibration: per (item, KV head, K/V) sum of squares over the item's first chunk.
struct CalibItem {
  size_t slab;       // byte offset of the (layer, seq) slab
  int src_row;       // first input row of the chunk
  int n;             // tokens in the chunk
};
struct CalibArgs {
  Geometry g;
  const uint16_t* k_in;
  const uint16_t* v_in;
  int n_items;
  CalibItem items[kMaxBatch];
};

// Body write (quantize into the qN_0 body), one work-group per (item, tile, KV head).
// Position p in [p0, p1): from input row src_row + (p - len_old) when p >= len_old (through the ring
// representation when the ring is q8_0), otherwise from ring slot p mod R.
// The same kernel writes q8_0 ring rows (dst_ring = 1: destination is the ring, source is the input).
struct WriteItem {
  size_t slab;
  int p0, p1;        // positions written
  int len_old;       // positions >= len_old come from the input
  int src_row;       // input row of position len_old
  int tile0;         // first position tile (p0 / 32)
  int wg_begin;      // first work-group of this item (prefix over items)
};
struct WriteArgs {
  Geometry g;
  const uint16_t* k_in;
  const uint16_t* v_in;
  int dst_ring;      // 0: body; 1: q8_0 ring
  int n_items;
  WriteItem items[kMaxBatch];
};

// A decode step's append (ring writes) and evict (body writes) in one launch; up to kStepBatch sequences.
constexpr int kStepBatch = 32;
struct StepRole {    // the members of WriteArgs, with room for kStepBatch items
  Geometry g;
  const uint16_t* k_in;
  const uint16_t* v_in;
  int dst_ring;
  int n_items;
  WriteItem items[kStepBatch];
};
struct StepArgs {
  StepRole ring;     // ring writes of the new tokens (dst_ring = 1)
  StepRole body;     // evict: ring rows requantized into the body (dst_ring = 0)
  int ring_wgs;      // work-groups of the ring writes (the rest are body writes)
};

// ---------------------------------------------------------------- decode side

struct DecodeSeq {
  size_t slab;
  int len, body_len;
  int n_body_splits, n_ring_splits;
  int ring_tile0;    // first position tile of the ring range (body_len / 32)
  // fused decode step (step != 0): the token appended at position app_pos (input row = sequence index; -1:
  // none) is written into the ring by the work-group of the last ring split, the ring rows [ev0, ev1) that
  // leave the window are requantized into the body by the work-group of the last body split, each before
  // it reads those tiles
  int app_pos, ev0, ev1;
  int last_tb;       // > 0: first tile of the last body split (the others share the tiles before it)
};
struct DecodeArgs {
  Geometry g;
  const uint16_t* q;           // [n_seqs][Hq][D] bf16
  float* out;                  // [n_seqs][Hq][D]
  float* partials;             // [n_seqs][Hkv][max_splits][8 * (D + 2)]
  const uint16_t* k_in;        // fused decode step: the appended K and V tokens [n_seqs][Hkv][D] bf16
  const uint16_t* v_in;
  int step;
  int n_seqs, n_q_heads, group, max_splits;
  float scale;                 // softmax scale
  DecodeSeq seqs[kMaxBatch];
};


constexpr int kGatherWaves = 4;    // waves per gather work-group (16 list entries per wave step)

// Gather decode over a list of positions of a row-layout cache (sparse decode), or over all positions
// (dense decode of a row-layout cache: positions == nullptr, entry i is position i).
struct GatherSeq {
  size_t slab;
  int len, body_len;
  int n_list;        // list entries of this sequence (budget, or len)
  int n_splits;      // work-groups per KV head
  int app_pos;       // fused sparse step: the body position written from input row (sequence index); -1: none
};
struct GatherArgs {
  Geometry g;
  const uint16_t* q;           // [n_seqs][Hq][D] bf16
  const int32_t* positions;    // [n_seqs][pos_stride] or nullptr
  int pos_stride;
  float* partials;             // [n_seqs][Hkv][max_splits][8 * (D + 2)]
  const uint16_t* k_in;        // fused sparse step: the appended K and V tokens [n_seqs][Hkv][D] bf16
  const uint16_t* v_in;
  int step;
  int n_seqs, n_q_heads, group, max_splits;
  float scale;
  GatherSeq seqs[kMaxBatch];
};

struct CombineArgs {
  float* out;
  const float* partials;
  int n_seqs, n_q_heads, n_kv_heads, group, head_dim, max_splits;
  int n_splits[kMaxBatch];
};

// ---------------------------------------------------------------- indexer (QSA)

// Pooled index keys of the newest n positions of each item's sequence: positions p0 .. p0 + n - 1 from input
// rows row0 .. row0 + n - 1 ([row][32 * pool] bf16); `begin` is the item's first position number over all items.
struct IndexWriteItem {
  size_t slab;
  int p0, n, row0, begin;
};
struct IndexWriteArgs {
  Geometry g;
  const uint16_t* key_in;
  int pool;
  int n_items;
  IndexWriteItem items[kMaxBatch];
};

// Selection of a budget of positions per sequence: the first m = len - recent positions are scored, k of them
// chosen, then the `recent` newest appended. Work-groups of kIndexChunk positions; ws_off: the sequence's part of the
// workspace (histogram, control words, keys, bitmap, candidates).
struct IndexSeq {
  size_t slab;
  size_t ws_off;
  int len, m, k;
  int n_wgs, wg_begin;
};
struct IndexArgs {
  Geometry g;
  const uint16_t* q;        // [n_seqs][32] bf16 index queries
  int32_t* out;             // [n_seqs][budget]
  uint8_t* ws;
  int budget;
  int n_seqs;
  IndexSeq seqs[kMaxBatch];
};
constexpr int kIndexChunk = 1024;      // positions per work-group of the selection kernels
constexpr int kIndexHistCopies = 4;    // copies of a sequence's 16,384-bin score histogram

// Workspace bytes of one sequence's selection with `n_wgs` work-groups: histogram copies, 16 control words,
// keys, bitmap, candidates.
inline size_t index_ws_seq_bytes(int n_wgs) {
  const size_t words = (size_t)kIndexHistCopies * (1 << 14) + 16 + (size_t)n_wgs * kIndexChunk +
                       (size_t)n_wgs * (kIndexChunk / 32);
  return round_up(words * 4 + (size_t)n_wgs * kIndexChunk * 8, 256);
}

// ---------------------------------------------------------------- multi-query attention (draft verification,
// chunked prefill)

// Queries of one sequence: positions q0 .. q0 + nq - 1 (q0 + nq <= len), rows row0 .. row0 + nq - 1 of q / out;
// query p attends to positions [0, p]. Blocks of 8 consecutive queries, each block and KV head split n_splits ways:
// with n_ring_splits == 0 the splits share the block's whole tile list (body tiles, then ring tiles), else
// n_splits - n_ring_splits body splits and n_ring_splits ring splits.
struct MqSeq {
  size_t slab;
  int len, body_len;
  int q0, nq, row0;
  int n_splits, n_ring_splits;
  int wg_begin;
};
struct MqArgs {
  Geometry g;
  const uint16_t* q;        // [rows][Hq][D] bf16
  float* out;               // [rows][Hq][D]
  float* partials;          // [rows][Hkv][max_splits][8 (D + 2)] (used when n_splits > 1)
  int n_seqs, n_q_heads, group, max_splits;
  float scale;
  MqSeq seqs[kMaxBatch];
};

// Launch wrappers (return the launch status). With non-null events e0 / e1 the launch records the kernel's
// start and end time in them (hipExtLaunchKernel: timestamps of the dispatch itself).
hipError_t launch_calibrate(const CalibArgs& a, int n_items, hipStream_t s, hipEvent_t e0 = nullptr,
                            hipEvent_t e1 = nullptr);
hipError_t launch_body_write(const WriteArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0 = nullptr,
                             hipEvent_t e1 = nullptr);
hipError_t launch_bf16_ring_write(const WriteArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0 = nullptr,
                                  hipEvent_t e1 = nullptr);
hipError_t launch_step_write(const StepArgs& a, int n_wgs, hipStream_t s, hipEvent_t e0 = nullptr,
                             hipEvent_t e1 = nullptr);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int grid_x, hipStream_t s, hipEvent_t e0 = nullptr,
                         hipEvent_t e1 = nullptr);
hipError_t launch_gather(const GatherArgs& a, int grid_x, hipStream_t s, hipEvent_t e0 = nullptr,
                         hipEvent_t e1 = nullptr);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_index_write(const IndexWriteArgs& a, int n_positions, hipStream_t s, hipEvent_t e0 = nullptr,
                              hipEvent_t e1 = nullptr);
hipError_t launch_mq(const MqArgs& a, int grid_x, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_mq_combine(const MqArgs& a, int rows, hipStream_t s, hipEvent_t e0 = nullptr,
                             hipEvent_t e1 = nullptr);
// The selection launches; e0 / e1 bracket the scoring and finishing launches.
hipError_t launch_index_select(const IndexArgs& a, int total_wgs, hipStream_t s, hipEvent_t e0 = nullptr,
                               hipEvent_t e1 = nullptr);

// The library's static scratch buffer (kvq_scratch.hip): kScratchBytes of device memory per GPU, for the
// entry points that take no workspace. scratch_device_ptr returns its device address on `device` (looked up
// once per device with that device current; later calls return the stored address).
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_device_ptr(int device, void** ptr);

// Plain or timed launch of a kernel with one by-value argument block.
template <typename K, typename A>
inline hipError_t launch_k(K kernel, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0, hipEvent_t e1, const A& a) {
  if (e0) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, a);
  else hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
