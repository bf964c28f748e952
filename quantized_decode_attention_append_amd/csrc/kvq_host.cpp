// Host side of the kvq C ABI: validation, per-(layer, sequence) bookkeeping, work planning and launches.
// Every entry point validates on the host before any HIP call; no exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_kernels.h"
#include "kvq_mq_plan.h"

using kvq::SlabLayout;

// Per-kernel launch timing (kvq_timing_enable): HIP event pairs recorded on the launch stream around
// each launch, read back by kvq_timing_read.
struct KernelTimes {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> used, spare;
};

struct kvq_cache {
  kvq_config cfg;
  bool timing = false;
  KernelTimes times[KVQ_KERNEL_COUNT];
  SlabLayout lay;
  uint8_t* arena;
  size_t arena_bytes;
  std::vector<int32_t> len, body_len;
  std::vector<uint8_t> calibrated;
  int n_cu = 256;            // compute units of the device (split planning)
  int device = 0;            // device current at kvq_cache_init (the arena's device)
  int idx(int layer, int seq) const { return layer * cfg.max_seqs + seq; }
  ~kvq_cache() {
    for (auto& t : times) {
      for (auto& e : t.used) { (void)hipEventDestroy(e.first); (void)hipEventDestroy(e.second); }
      for (auto& e : t.spare) { (void)hipEventDestroy(e.first); (void)hipEventDestroy(e.second); }
    }
  }
};

namespace {

thread_local std::string g_err = "no error";

kvq_status fail(kvq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvq_status fail(kvq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kMaxTimedLaunches = 1 << 16;   // per kernel kind between two kvq_timing_enable calls

// Run `launch(e0, e1)`; with timing on, e0 / e1 are events that the launch fills with the kernel's start
// and end time (null otherwise).
template <typename F>
hipError_t timed(kvq_cache* c, int kind, hipStream_t stream, F launch) {
  (void)stream;
  if (!c->timing || c->times[kind].used.size() >= kMaxTimedLaunches) return launch(nullptr, nullptr);
  KernelTimes& t = c->times[kind];
  std::pair<hipEvent_t, hipEvent_t> ev;
  if (!t.spare.empty()) {
    ev = t.spare.back();
    t.spare.pop_back();
  } else {
    hipError_t e = hipEventCreate(&ev.first);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&ev.second);
    if (e != hipSuccess) { (void)hipEventDestroy(ev.first); return e; }
  }
  hipError_t e = launch(ev.first, ev.second);
  if (e == hipSuccess) t.used.push_back(ev);
  else t.spare.push_back(ev);
  return e;
}

SlabLayout layout_of(const kvq_config& c) {
  return kvq::slab_layout(c.capacity, c.n_kv_heads, c.head_dim, c.k_bits, c.v_bits, c.kvarn, c.tail_len,
                          c.tail_slack, c.tail_dtype, c.index_dim > 0 ? 1 : 0, c.k_min, c.v_min,
                          c.layout == KVQ_LAYOUT_ROWS ? 1 : 0);
}

kvq_status validate(const kvq_config* c) {
  if (!c) return fail(KVQ_E_INVALID, "config is NULL");
  if (c->n_layers < 1) return fail(KVQ_E_INVALID, "n_layers must be >= 1 (got %d)", c->n_layers);
  if (c->max_seqs < 1) return fail(KVQ_E_INVALID, "max_seqs must be >= 1 (got %d)", c->max_seqs);
  if (c->capacity < 1 || c->capacity > (1 << 28))
    return fail(KVQ_E_INVALID, "capacity must be in [1, 2^28] (got %d)", c->capacity);
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVQ_E_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c->n_q_heads,
                c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > kvq::kPartialHeads)
    return fail(KVQ_E_INVALID, "query group n_q_heads / n_kv_heads must be <= 8 (got %d)",
                c->n_q_heads / c->n_kv_heads);
  if (c->head_dim != 256) return fail(KVQ_E_INVALID, "head_dim must be 256 (got %d)", c->head_dim);
  if (c->k_bits < 2 || c->k_bits > 8 || c->v_bits < 2 || c->v_bits > 8)
    return fail(KVQ_E_INVALID, "k_bits and v_bits must be in [2, 8] (got %d, %d)", c->k_bits, c->v_bits);
  if (c->kvarn != 0 && c->kvarn != 1) return fail(KVQ_E_INVALID, "kvarn must be 0 or 1");
  if ((c->k_min != 0 && c->k_min != 1) || (c->v_min != 0 && c->v_min != 1))
    return fail(KVQ_E_INVALID, "k_min and v_min must be 0 or 1 (got %d, %d)", c->k_min, c->v_min);
  if ((c->k_min || c->v_min) && c->layout != KVQ_LAYOUT_TILES)
    return fail(KVQ_E_INVALID, "qN_1 bodies (k_min / v_min) need KVQ_LAYOUT_TILES");
  if (c->k_axis != 0 && c->k_axis != 1) return fail(KVQ_E_INVALID, "k_axis must be 0 or 1 (got %d)", c->k_axis);
  if (c->k_axis && (c->layout != KVQ_LAYOUT_TILES || c->tail_len < 1 || c->tail_slack < kvq::kTile))
    return fail(KVQ_E_INVALID, "token-axis K (k_axis) needs KVQ_LAYOUT_TILES, tail_len >= 1 and tail_slack >= 32");
  if (c->tail_len < 0 || c->tail_slack < 0) return fail(KVQ_E_INVALID, "tail_len and tail_slack must be >= 0");
  if (c->layout != KVQ_LAYOUT_TILES && c->layout != KVQ_LAYOUT_ROWS)
    return fail(KVQ_E_INVALID, "layout must be KVQ_LAYOUT_TILES or KVQ_LAYOUT_ROWS (got %d)", c->layout);
  if (c->index_dim != 0) {
    const int p = c->index_pool;
    if (p != 1 && p != 2 && p != 4 && p != 8 && p != 16)
      return fail(KVQ_E_INVALID, "index_pool must be 1, 2, 4, 8 or 16 (got %d)", p);
    if (c->index_dim != kvq::kIndexWidth * p)
      return fail(KVQ_E_INVALID, "index_dim must be 32 x index_pool (got %d with pool %d)", c->index_dim, p);
  }
  if (c->tail_len > 0) {
    if (c->tail_dtype != KVQ_TAIL_BF16 && c->tail_dtype != KVQ_TAIL_Q8_0 && c->tail_dtype != KVQ_TAIL_F16)
      return fail(KVQ_E_INVALID, "tail_dtype must be KVQ_TAIL_BF16, KVQ_TAIL_Q8_0 or KVQ_TAIL_F16 when tail_len > 0");
    const long r = (long)c->tail_len + c->tail_slack;
    if (r % kvq::kTile != 0) return fail(KVQ_E_INVALID, "tail_len + tail_slack must be a multiple of 32 (got %ld)", r);
    if (r > (1 << 24)) return fail(KVQ_E_INVALID, "tail_len + tail_slack too large");
  }
  return KVQ_OK;
}

kvq::Geometry geometry(const kvq_cache* c) {
  kvq::Geometry g{};
  g.arena = c->arena;
  g.slab_bytes = c->lay.slab;
  g.k_body = c->lay.k_body;
  g.v_body = c->lay.v_body;
  g.k_ring = c->lay.k_ring;
  g.v_ring = c->lay.v_ring;
  g.sigma = c->lay.sigma;
  g.index = c->lay.index;
  g.cap32 = c->lay.cap32;
  g.row_k = c->lay.row_k;
  g.row_v = c->lay.row_v;
  g.tile_k = kvq::kTile * c->lay.row_k;
  g.tile_v = kvq::kTile * c->lay.row_v;
  g.ring_row_k = c->lay.ring_row_k;
  g.ring_tile_k = kvq::kTile * c->lay.ring_row_k;
  g.ring_tile_v = kvq::kTile * c->lay.ring_row_v;
  g.ring_row_v = c->lay.ring_row_v;
  g.ring_slots = c->lay.ring_slots;
  g.layout = c->cfg.layout;
  g.n_kv_heads = c->cfg.n_kv_heads;
  g.head_dim = c->cfg.head_dim;
  g.k_bits = c->cfg.k_bits;
  g.v_bits = c->cfg.v_bits;
  g.kvarn = c->cfg.kvarn;
  g.tail_dtype = c->cfg.tail_len > 0 ? c->cfg.tail_dtype : 0;
  g.k_min = c->cfg.k_min;
  g.v_min = c->cfg.v_min;
  g.k_axis = c->cfg.k_axis;
  return g;
}

size_t slab_offset(const kvq_cache* c, int layer, int seq) {
  return ((size_t)layer * c->cfg.max_seqs + seq) * c->lay.slab;
}

kvq_status check_seqs(const kvq_cache* c, int layer, int n_seqs, const int32_t* ids) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVQ_E_INVALID, "layer %d out of range", layer);
  if (n_seqs < 1 || n_seqs > KVQ_MAX_BATCH)
    return fail(KVQ_E_INVALID, "n_seqs must be in [1, %d] (got %d)", KVQ_MAX_BATCH, n_seqs);
  if (!ids) return fail(KVQ_E_INVALID, "seq_ids is NULL");
  for (int i = 0; i < n_seqs; ++i) {
    if (ids[i] < 0 || ids[i] >= c->cfg.max_seqs) return fail(KVQ_E_INVALID, "seq id %d out of range", ids[i]);
    for (int j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return fail(KVQ_E_INVALID, "seq id %d repeated", ids[i]);
  }
  return KVQ_OK;
}

int tiles_of(int p0, int p1) { return p1 > p0 ? (p1 - 1) / kvq::kTile - p0 / kvq::kTile + 1 : 0; }

// Split planning. The decode kernel runs one 8-wave work-group per split and the plan aims at about one
// work-group per CU: each (sequence, body|ring) segment gets a share of the CU budget proportional to
// its tiles (at least one), leftover work-groups go to the segments with the most tiles per work-group.
constexpr int kMaxWgBudget = 1024;
// Decode work-groups planned per CU: two 8-wave work-groups are co-resident on a CU (64 KiB of LDS and at most
// 128 VGPRs each), so the plan fills both slots.
#ifndef KVQ_DECODE_WGS_PER_CU
#define KVQ_DECODE_WGS_PER_CU 1
#endif
constexpr int kDecodeWgsPerCu = KVQ_DECODE_WGS_PER_CU;
constexpr int kMinTilesPerWg = 4;
// Ring work-groups per sequence that multi-query decode plans outside the per-head budget (at most).
constexpr int kRingExtra = 2;

constexpr size_t kPartialFloats(int d) { return (size_t)kvq::kPartialHeads * (d + 2); }

struct SplitPlan {
  int max_splits;   // per (sequence, KV head)
  int total_wgs;
};

// allow_ring_extra: when the sequences are many against the per-head budget (as the entries of multi-query
// decode can be), their short ring segments get work-groups on top of the budget instead of taking most of it
// from the body segments.
SplitPlan plan_splits(const kvq_cache* c, int n_seqs, const int* len, const int* body_len, kvq::DecodeSeq* out,
                      bool allow_ring_extra = false) {
  const int hk = c->cfg.n_kv_heads;
  int budget_h = std::max(1, std::min(kDecodeWgsPerCu * c->n_cu, kMaxWgBudget) / hk);   // work-groups per KV head
  // Cost of a tile in a work-group's time: a qN_0 tile (body or q8_0 ring) is decode- and MFMA-bound, a bf16
  // ring tile carries 2.7x the bytes of a K6/V5 tile with little decode and no prefetch: it counts double.
  const double ring_w = c->cfg.tail_dtype == KVQ_TAIL_Q8_0 ? 1.0 : 2.0;
  int tiles[2 * KVQ_MAX_BATCH], nwg[2 * KVQ_MAX_BATCH];
  double wt[2 * KVQ_MAX_BATCH];
  double total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    tiles[2 * i] = (body_len[i] + kvq::kTile - 1) / kvq::kTile;
    tiles[2 * i + 1] =
        len[i] > body_len[i] ? (len[i] + kvq::kTile - 1) / kvq::kTile - body_len[i] / kvq::kTile : 0;
    wt[2 * i] = tiles[2 * i];
    wt[2 * i + 1] = ring_w * tiles[2 * i + 1];
    total += wt[2 * i] + wt[2 * i + 1];
  }
  // short contexts: at least ~kMinTilesPerWg tiles of cost per work-group (fewer, fuller work-groups and fewer
  // partials to merge; measured on the 4k single-layer workload)
  budget_h = std::min(budget_h, std::max(1, (int)(total / kMinTilesPerWg)));
  const bool ring_extra = allow_ring_extra && 4 * n_seqs > budget_h;
  double shared = total;   // the cost that shares the budget
  if (ring_extra) {
    shared = 0;
    for (int i = 0; i < n_seqs; ++i) shared += wt[2 * i];
  }
  const double per_wg = std::max(shared / budget_h, 1.0);
  int used = 0;
  for (int k = 0; k < 2 * n_seqs; ++k) {
    if (ring_extra && (k & 1)) {   // outside the budget: about one body work-group's cost each, at most kRingExtra
      nwg[k] = tiles[k] ? std::min({tiles[k], kRingExtra, std::max(1, (int)(wt[k] / per_wg + 0.5))}) : 0;
      continue;
    }
    nwg[k] = tiles[k] ? std::max(1, (int)(budget_h * wt[k] / std::max(shared, 1.0))) : 0;
    nwg[k] = std::min(nwg[k], tiles[k]);
    used += nwg[k];
  }
  for (; used < budget_h; ++used) {   // leftover: the segment with the most cost per work-group
    int best = -1;
    double best_r = 0.0;
    for (int k = 0; k < 2 * n_seqs; ++k)
      if (!(ring_extra && (k & 1)) && nwg[k] && nwg[k] < tiles[k] && wt[k] / nwg[k] > best_r) {
        best_r = wt[k] / nwg[k];
        best = k;
      }
    if (best < 0) break;
    ++nwg[best];
  }
  SplitPlan p{1, 0};
  for (int i = 0; i < n_seqs; ++i) {
    if (out) {
      out[i].len = len[i];
      out[i].body_len = body_len[i];
      out[i].n_body_splits = nwg[2 * i];
      out[i].n_ring_splits = nwg[2 * i + 1];
      out[i].ring_tile0 = body_len[i] / kvq::kTile;
    }
    p.max_splits = std::max(p.max_splits, nwg[2 * i] + nwg[2 * i + 1]);
    p.total_wgs += hk * (nwg[2 * i] + nwg[2 * i + 1]);
  }
  return p;
}

// Gather decode: list entries per work-group are at least kGatherMin (one 16-entry step for each of its
// waves); up to two work-groups per CU over all (sequence, KV head) pairs.
constexpr int kGatherMin = 16 * kvq::kGatherWaves;
int gather_budget_h(const kvq_cache* c) {
  return std::max(1, std::min(2 * c->n_cu, kvq::kMaxSplits) / c->cfg.n_kv_heads);
}
int plan_gather(const kvq_cache* c, int n_seqs, const int* n_list, kvq::GatherSeq* out, int* total_wgs) {
  long total = 0;
  for (int i = 0; i < n_seqs; ++i) total += n_list[i];
  const int budget = gather_budget_h(c);
  int max_splits = 1;
  *total_wgs = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int by_size = (n_list[i] + kGatherMin - 1) / kGatherMin;
    const int by_share = (int)std::max(1L, (long)budget * n_list[i] / std::max(total, 1L));
    const int ns = std::max(1, std::min(by_size, by_share));
    out[i].n_splits = ns;
    max_splits = std::max(max_splits, ns);
    *total_wgs += c->cfg.n_kv_heads * ns;
  }
  return max_splits;
}

kvq_status launch_combine_for(kvq_cache* c, int n_seqs, const int* n_splits, int max_splits, float* out,
                              void* workspace, hipStream_t stream) {
  kvq::CombineArgs cb{};
  cb.out = out;
  cb.partials = (const float*)workspace;
  cb.n_seqs = n_seqs;
  cb.n_q_heads = c->cfg.n_q_heads;
  cb.n_kv_heads = c->cfg.n_kv_heads;
  cb.group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  cb.head_dim = c->cfg.head_dim;
  cb.max_splits = max_splits;
  for (int i = 0; i < n_seqs; ++i) cb.n_splits[i] = n_splits[i];
  hipError_t e = timed(c, KVQ_KERNEL_COMBINE, stream, [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_combine(cb, stream, e0, e1); });
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return KVQ_OK;
}

// The gather path shared by sparse decode and dense decode of a row-layout cache. positions: device
// [n_seqs][pos_stride] or nullptr (entry i = position i, n_list[i] = len). With k_in / v_in (a fused sparse
// step of a cache without a ring) the launch first appends one token per sequence at its current length.
kvq_status run_gather(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q_bf16,
                      const int32_t* positions, int pos_stride, const int* n_list, float* out, float softmax_scale,
                      void* workspace, size_t ws_bytes, void* stream, const void* k_in = nullptr,
                      const void* v_in = nullptr) {
  kvq::GatherArgs a{};
  a.g = geometry(c);
  int total_wgs = 0;
  const int max_splits = plan_gather(c, n_seqs, n_list, a.seqs, &total_wgs);
  const size_t need = (size_t)n_seqs * c->cfg.n_kv_heads * max_splits * kPartialFloats(c->cfg.head_dim) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  int n_splits[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    const int app = k_in ? 1 : 0;
    a.seqs[i].slab = slab_offset(c, layer, seq_ids[i]);
    a.seqs[i].len = c->len[k] + app;
    a.seqs[i].body_len = c->body_len[k] + app;
    a.seqs[i].n_list = n_list[i];
    a.seqs[i].app_pos = app ? c->len[k] : -1;
    n_splits[i] = a.seqs[i].n_splits;
  }
  a.q = (const uint16_t*)q_bf16;
  a.k_in = (const uint16_t*)k_in;
  a.v_in = (const uint16_t*)v_in;
  a.step = k_in ? 1 : 0;
  a.positions = positions;
  a.pos_stride = pos_stride;
  a.partials = (float*)workspace;
  a.n_seqs = n_seqs;
  a.n_q_heads = c->cfg.n_q_heads;
  a.group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  a.max_splits = max_splits;
  a.scale = softmax_scale > 0 ? softmax_scale : 1.0f / std::sqrt((float)c->cfg.head_dim);
  hipError_t e = timed(c, KVQ_KERNEL_GATHER, (hipStream_t)stream,
                       [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_gather(a, total_wgs, (hipStream_t)stream, e0, e1); });
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  if (k_in) {
    for (int i = 0; i < n_seqs; ++i) {
      const int k = c->idx(layer, seq_ids[i]);
      c->len[k] += 1;
      c->body_len[k] = c->len[k];
    }
  }
  return launch_combine_for(c, n_seqs, n_splits, max_splits, out, workspace, (hipStream_t)stream);
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return g_err.c_str(); }

kvq_status kvq_timing_enable(kvq_cache* c, int32_t enable) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (enable != 0 && enable != 1) return fail(KVQ_E_INVALID, "enable must be 0 or 1");
  for (auto& t : c->times) {   // records of earlier launches are dropped (their events are reused)
    t.spare.insert(t.spare.end(), t.used.begin(), t.used.end());
    t.used.clear();
  }
  c->timing = enable != 0;
  return KVQ_OK;
}

kvq_status kvq_timing_read(kvq_cache* c, int32_t kernel, double* total_ms, int32_t* launches) {
  if (!c || !total_ms || !launches) return fail(KVQ_E_INVALID, "cache/total_ms/launches is NULL");
  if (kernel < 0 || kernel >= KVQ_KERNEL_COUNT) return fail(KVQ_E_INVALID, "unknown kernel kind %d", kernel);
  double sum = 0.0;
  for (const auto& ev : c->times[kernel].used) {
    hipError_t e = hipEventSynchronize(ev.second);
    if (e != hipSuccess) return hip_fail(e, "timing event");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, ev.first, ev.second);
    if (e != hipSuccess) return hip_fail(e, "timing event");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int32_t)c->times[kernel].used.size();
  return KVQ_OK;
}

kvq_status kvq_config_validate(const kvq_config* cfg) { return validate(cfg); }

size_t kvq_cache_bytes(const kvq_config* cfg) {
  if (validate(cfg) != KVQ_OK) return 0;
  return (size_t)cfg->n_layers * cfg->max_seqs * layout_of(*cfg).slab;
}

kvq_status kvq_region(const kvq_config* cfg, int32_t layer, int32_t seq, int32_t region, size_t* offset,
                      size_t* bytes) {
  kvq_status s = validate(cfg);
  if (s != KVQ_OK) return s;
  if (!offset || !bytes) return fail(KVQ_E_INVALID, "offset/bytes is NULL");
  if (layer < 0 || layer >= cfg->n_layers || seq < 0 || seq >= cfg->max_seqs)
    return fail(KVQ_E_INVALID, "layer/seq out of range");
  const SlabLayout L = layout_of(*cfg);
  const size_t base = ((size_t)layer * cfg->max_seqs + seq) * L.slab;
  switch (region) {
    case KVQ_REGION_K_BODY: *offset = base + L.k_body; *bytes = L.k_body_sz; break;
    case KVQ_REGION_V_BODY: *offset = base + L.v_body; *bytes = L.v_body_sz; break;
    case KVQ_REGION_K_RING: *offset = base + L.k_ring; *bytes = L.k_ring_sz; break;
    case KVQ_REGION_V_RING: *offset = base + L.v_ring; *bytes = L.v_ring_sz; break;
    case KVQ_REGION_SIGMA: *offset = base + L.sigma; *bytes = L.sigma_sz; break;
    case KVQ_REGION_SLAB: *offset = base; *bytes = L.slab; break;
    case KVQ_REGION_INDEX: *offset = base + L.index; *bytes = L.index_sz; break;
    default: return fail(KVQ_E_INVALID, "unknown region %d", region);
  }
  return KVQ_OK;
}

kvq_status kvq_cache_init(const kvq_config* cfg, void* dev_arena, size_t arena_bytes, void* stream,
                          kvq_cache** out) {
  kvq_status s = validate(cfg);
  if (s != KVQ_OK) return s;
  if (!out) return fail(KVQ_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!dev_arena) return fail(KVQ_E_INVALID, "arena is NULL");
  if (((uintptr_t)dev_arena) % 256 != 0) return fail(KVQ_E_INVALID, "arena must be 256-byte aligned");
  const size_t need = kvq_cache_bytes(cfg);
  if (arena_bytes < need) return fail(KVQ_E_SIZE, "arena has %zu bytes, needs %zu", arena_bytes, need);
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_E_INVALID, "out of host memory");
  c->cfg = *cfg;
  c->lay = layout_of(*cfg);
  c->arena = (uint8_t*)dev_arena;
  c->arena_bytes = arena_bytes;
  const size_t n = (size_t)cfg->n_layers * cfg->max_seqs;
  c->len.assign(n, 0);
  c->body_len.assign(n, 0);
  c->calibrated.assign(n, 0);
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
    c->n_cu = ncu;
  c->device = dev;
  {   // set-up of the static scratch on this device (kvq_decode_attn_noalloc); a failure here is reported by
      // that entry point, which looks the address up again
    void* p = nullptr;
    (void)kvq::scratch_device_ptr(dev, &p);
  }
  hipError_t e = kvq::launch_fill_zero(dev_arena, need, (hipStream_t)stream);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "zero-fill of the arena");
  }
  *out = c;
  return KVQ_OK;
}

void kvq_cache_destroy(kvq_cache* cache) { delete cache; }

kvq_status kvq_seq_truncate(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const int32_t* new_len) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (!new_len) return fail(KVQ_E_INVALID, "new_len is NULL");
  for (int i = 0; i < n_seqs; ++i) {   // every sequence is checked before any is changed
    const int k = c->idx(layer, seq_ids[i]);
    if (new_len[i] < 0 || new_len[i] > c->len[k])
      return fail(KVQ_E_INVALID, "seq %d: new length %d outside [0, %d]", seq_ids[i], new_len[i], c->len[k]);
    if (new_len[i] < c->body_len[k])
      return fail(KVQ_E_STATE, "seq %d: new length %d would drop body rows (body_len %d)", seq_ids[i], new_len[i],
                  c->body_len[k]);
  }
  // ring writes read-modify-write their slot, so the dropped rows need no clearing
  for (int i = 0; i < n_seqs; ++i) c->len[c->idx(layer, seq_ids[i])] = new_len[i];
  return KVQ_OK;
}

kvq_status kvq_seq_reset(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, void* stream) {
  if (!c) return fail(KVQ_E_INVALID, "cache is NULL");
  if (layer < -1 || layer >= c->cfg.n_layers) return fail(KVQ_E_INVALID, "layer %d out of range", layer);
  kvq_status s = check_seqs(c, layer < 0 ? 0 : layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  const int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->cfg.n_layers : layer + 1;
  for (int l = l0; l < l1; ++l)
    for (int i = 0; i < n_seqs; ++i) {
      hipError_t e = kvq::launch_fill_zero(c->arena + slab_offset(c, l, seq_ids[i]), c->lay.slab, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "zero-fill of a slab");
      const int k = c->idx(l, seq_ids[i]);
      c->len[k] = c->body_len[k] = 0;
      c->calibrated[k] = 0;
    }
  return KVQ_OK;
}

kvq_status kvq_seq_lengths(const kvq_cache* c, int32_t layer, int32_t seq, int32_t* len, int32_t* body_len) {
  if (!c || !len || !body_len) return fail(KVQ_E_INVALID, "NULL argument");
  if (layer < 0 || layer >= c->cfg.n_layers || seq < 0 || seq >= c->cfg.max_seqs)
    return fail(KVQ_E_INVALID, "layer/seq out of range");
  *len = c->len[c->idx(layer, seq)];
  *body_len = c->body_len[c->idx(layer, seq)];
  return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_cache* c, int32_t n_seqs, int32_t max_len) {
  if (!c || n_seqs < 1 || max_len < 1) return 0;
  // splits per (sequence, KV head) never exceed the tiles of a sequence (+1 for the body/ring boundary
  // tile) nor the per-head work-group budget
  const long tiles = (max_len + kvq::kTile - 1) / kvq::kTile + 1;
  long splits = std::min<long>(
      tiles, std::max(1, std::min(kDecodeWgsPerCu * c->n_cu, kMaxWgBudget) / c->cfg.n_kv_heads) + kRingExtra);
  // the gather path (sparse decode, and dense decode of a row-layout cache)
  const long gsplits = std::min<long>((max_len + kGatherMin - 1) / kGatherMin, gather_budget_h(c));
  splits = std::max(splits, std::max(1L, gsplits));
  return (size_t)n_seqs * c->cfg.n_kv_heads * splits * kPartialFloats(c->cfg.head_dim) * sizeof(float);
}

kvq_status kvq_append(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                      const void* k_bf16, const void* v_bf16, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (!n_new) return fail(KVQ_E_INVALID, "n_new is NULL");
  long total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (n_new[i] < 0) return fail(KVQ_E_INVALID, "n_new[%d] is negative", i);
    const int k = c->idx(layer, seq_ids[i]);
    if ((long)c->len[k] + n_new[i] > c->cfg.capacity)
      return fail(KVQ_E_CAPACITY, "seq %d: %d + %d positions exceed capacity %d", seq_ids[i], c->len[k], n_new[i],
                  c->cfg.capacity);
    total += n_new[i];
  }
  if (total == 0) return KVQ_OK;
  if (!k_bf16 || !v_bf16) return fail(KVQ_E_INVALID, "k/v input is NULL");

  const kvq::Geometry g = geometry(c);
  const hipStream_t st = (hipStream_t)stream;
  const int W = c->cfg.tail_len;
  const int R = c->lay.ring_slots;

  kvq::CalibArgs ca{};
  ca.g = g;
  ca.k_in = (const uint16_t*)k_bf16;
  ca.v_in = (const uint16_t*)v_bf16;
  kvq::WriteArgs body{}, ring{}, ring2{};
  body.g = ring.g = ring2.g = g;
  body.k_in = ring.k_in = ring2.k_in = (const uint16_t*)k_bf16;
  body.v_in = ring.v_in = ring2.v_in = (const uint16_t*)v_bf16;
  body.dst_ring = 0;
  ring.dst_ring = ring2.dst_ring = 1;
  int body_wgs = 0, ring_wgs = 0, ring2_wgs = 0;
  std::vector<int> new_len(n_seqs), new_body(n_seqs);

  int row = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    const int n = n_new[i];
    const int len = c->len[k], bl = c->body_len[k];
    const size_t slab = slab_offset(c, layer, seq_ids[i]);
    new_len[i] = len + n;
    new_body[i] = bl;
    if (n == 0) continue;
    if (c->cfg.kvarn && !c->calibrated[k]) ca.items[ca.n_items++] = kvq::CalibItem{slab, row, n};
    int b0, b1, r0 = 0, r1 = 0;
    if (W == 0) {
      b0 = len;
      b1 = len + n;
      new_body[i] = len + n;
    } else {
      // token-axis K: the body grows by whole tiles (a tile's K blocks need all its positions)
      const int over = len + n - R;
      const int nb = std::max(bl, c->cfg.k_axis ? (over > 0 ? (over + kvq::kTile - 1) / kvq::kTile * kvq::kTile : 0)
                                               : over);
      b0 = bl;
      b1 = nb;
      r0 = std::max(len, nb);
      r1 = len + n;
      new_body[i] = nb;
    }
    if (b1 > b0) {
      kvq::WriteItem& it = body.items[body.n_items++];
      it = kvq::WriteItem{slab, b0, b1, len, row, b0 / kvq::kTile, body_wgs};
      body_wgs += tiles_of(b0, b1);
    }
    if (r1 > r0) {
      // A ring write of up to R positions spans at most R/32 + 1 position tiles; when it does, its first
      // and last tiles land in the same ring tile. The q8_0 ring updates V tiles by read-modify-write, so
      // the last tile then goes to a second, stream-ordered launch.
      int r_split = r1;
      if (c->cfg.tail_dtype == KVQ_TAIL_Q8_0 && tiles_of(r0, r1) > R / kvq::kTile)
        r_split = (r1 - 1) / kvq::kTile * kvq::kTile;
      kvq::WriteItem& it = ring.items[ring.n_items++];
      it = kvq::WriteItem{slab, r0, r_split, len, row, r0 / kvq::kTile, ring_wgs};
      ring_wgs += tiles_of(r0, r_split);
      if (r_split < r1) {
        kvq::WriteItem& it2 = ring2.items[ring2.n_items++];
        it2 = kvq::WriteItem{slab, r_split, r1, len, row, r_split / kvq::kTile, ring2_wgs};
        ring2_wgs += tiles_of(r_split, r1);
      }
    }
    row += n;
  }

  hipError_t e;
  if (ca.n_items) {
    e = timed(c, KVQ_KERNEL_APPEND, st, [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_calibrate(ca, ca.n_items, st, e0, e1); });
    if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  }
  if (body_wgs) {
    e = timed(c, KVQ_KERNEL_APPEND, st, [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_body_write(body, body_wgs, st, e0, e1); });
    if (e != hipSuccess) return hip_fail(e, "body write launch");
  }
  if (ring_wgs) {
    e = timed(c, KVQ_KERNEL_APPEND, st, [&](hipEvent_t e0, hipEvent_t e1) {
      return (c->cfg.tail_dtype != KVQ_TAIL_Q8_0) ? kvq::launch_bf16_ring_write(ring, ring_wgs, st, e0, e1)
                                                  : kvq::launch_body_write(ring, ring_wgs, st, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(e, "ring write launch");
  }
  if (ring2_wgs) {
    e = timed(c, KVQ_KERNEL_APPEND, st, [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_body_write(ring2, ring2_wgs, st, e0, e1); });
    if (e != hipSuccess) return hip_fail(e, "ring write launch");
  }
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    if (n_new[i] > 0 && c->cfg.kvarn) c->calibrated[k] = 1;
    c->len[k] = new_len[i];
    c->body_len[k] = new_body[i];
  }
  return KVQ_OK;
}

kvq_status kvq_tail_evict(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  const int W = c->cfg.tail_len;
  if (W == 0) return KVQ_OK;
  kvq::WriteArgs body{};
  body.g = geometry(c);
  body.dst_ring = 0;
  int wgs = 0;
  std::vector<int> target(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    const int len = c->len[k], bl = c->body_len[k];
    int t = len - W;
    if (c->cfg.k_axis) t = t > 0 ? t / kvq::kTile * kvq::kTile : 0;   // whole tiles only
    target[i] = std::max(bl, t);
    if (target[i] > bl) {
      kvq::WriteItem& it = body.items[body.n_items++];
      it = kvq::WriteItem{slab_offset(c, layer, seq_ids[i]), bl, target[i], len, 0, bl / kvq::kTile, wgs};
      wgs += tiles_of(bl, target[i]);
    }
  }
  if (wgs) {
    hipError_t e = timed(c, KVQ_KERNEL_EVICT, (hipStream_t)stream,
                         [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_body_write(body, wgs, (hipStream_t)stream, e0, e1); });
    if (e != hipSuccess) return hip_fail(e, "evict launch");
  }
  for (int i = 0; i < n_seqs; ++i) c->body_len[c->idx(layer, seq_ids[i])] = target[i];
  return KVQ_OK;
}

kvq_status kvq_append_evict(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                            const void* k_bf16, const void* v_bf16, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (!n_new) return fail(KVQ_E_INVALID, "n_new is NULL");
  const int W = c->cfg.tail_len;
  const int R = c->lay.ring_slots;
  // One launch only for a pure ring write plus an evict of rows that were in the ring before the call:
  // then the ring writes and the body writes touch disjoint bytes and neither reads what the other writes.
  bool fuse = W > 0 && n_seqs <= kvq::kStepBatch && !c->cfg.k_axis;
  long total = 0;
  for (int i = 0; i < n_seqs && fuse; ++i) {
    if (n_new[i] < 0) { fuse = false; break; }   // reported by kvq_append
    const int k = c->idx(layer, seq_ids[i]);
    const int len = c->len[k], bl = c->body_len[k], n = n_new[i];
    total += n;
    if ((long)len + n > c->cfg.capacity) fuse = false;                      // reported by kvq_append
    else if (n > 0 && c->cfg.kvarn && !c->calibrated[k]) fuse = false;       // calibration comes first
    else if (len + n - bl > R) fuse = false;                                 // the append would evict itself
    else if (std::max(bl, len + n - W) > len) fuse = false;                  // would evict rows of this call
    else if (c->cfg.tail_dtype == KVQ_TAIL_Q8_0 && tiles_of(len, len + n) > R / kvq::kTile) fuse = false;
  }
  if (!fuse || total == 0 || !k_bf16 || !v_bf16) {
    s = kvq_append(c, layer, n_seqs, seq_ids, n_new, k_bf16, v_bf16, stream);
    return s != KVQ_OK ? s : kvq_tail_evict(c, layer, n_seqs, seq_ids, stream);
  }
  kvq::StepArgs a{};
  a.ring.g = a.body.g = geometry(c);
  a.ring.k_in = a.body.k_in = (const uint16_t*)k_bf16;
  a.ring.v_in = a.body.v_in = (const uint16_t*)v_bf16;
  a.ring.dst_ring = 1;
  a.body.dst_ring = 0;
  int ring_wgs = 0, body_wgs = 0, row = 0;
  std::vector<int> target(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    const int len = c->len[k], bl = c->body_len[k], n = n_new[i];
    const size_t slab = slab_offset(c, layer, seq_ids[i]);
    target[i] = std::max(bl, len + n - W);
    if (n > 0) {
      a.ring.items[a.ring.n_items++] = kvq::WriteItem{slab, len, len + n, len, row, len / kvq::kTile, ring_wgs};
      ring_wgs += tiles_of(len, len + n);
    }
    if (target[i] > bl) {
      a.body.items[a.body.n_items++] = kvq::WriteItem{slab, bl, target[i], len + n, 0, bl / kvq::kTile, body_wgs};
      body_wgs += tiles_of(bl, target[i]);
    }
    row += n;
  }
  a.ring_wgs = ring_wgs;
  if (ring_wgs + body_wgs) {
    hipError_t e = timed(c, KVQ_KERNEL_APPEND_EVICT, (hipStream_t)stream, [&](hipEvent_t e0, hipEvent_t e1) {
      return kvq::launch_step_write(a, ring_wgs + body_wgs, (hipStream_t)stream, e0, e1);
    });
    if (e != hipSuccess) return hip_fail(e, "append/evict launch");
  }
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    c->len[k] += n_new[i];
    c->body_len[k] = target[i];
  }
  return KVQ_OK;
}

extern "C++" {   // internal helpers between the exported entry points: C++ linkage
namespace {

// Dense decode of n entries, entry i reading sequence ids[i] over positions [0, len[i]) (its body range
// [0, min(body_len, len[i])) and the ring rows after it): the query and output rows follow the entries.
kvq_status run_mq(kvq_cache* c, int layer, int n, const int32_t* ids, const int* q0, const int* nq, const void* q_bf16,
                  float* out, float softmax_scale, void* workspace, size_t ws_bytes, void* stream,
                  bool balance = false);

kvq_status run_decode(kvq_cache* c, int32_t layer, int n, const int32_t* ids, const int* len, const void* q_bf16,
                      float* out, float softmax_scale, void* workspace, size_t ws_bytes, void* stream,
                      bool ring_extra = false) {
  if (c->cfg.layout == KVQ_LAYOUT_ROWS)
    return run_gather(c, layer, n, ids, q_bf16, nullptr, 0, len, out, softmax_scale, workspace, ws_bytes, stream);
  if (c->cfg.k_min || c->cfg.v_min || c->cfg.k_axis) {
    // qN_1 bodies and token-axis K are read by the multi-query kernel (its cooperative tile decode carries the
    // block minima and the per-channel K scales): each entry is a block of one query at the last of its positions
    int q0[KVQ_MAX_BATCH], nq[KVQ_MAX_BATCH];
    for (int i = 0; i < n; ++i) {
      q0[i] = len[i] - 1;
      nq[i] = 1;
    }
    return run_mq(c, layer, n, ids, q0, nq, q_bf16, out, softmax_scale, workspace, ws_bytes, stream);
  }
  int bl[KVQ_MAX_BATCH];
  for (int i = 0; i < n; ++i) bl[i] = std::min(c->body_len[c->idx(layer, ids[i])], len[i]);
  kvq::DecodeArgs a{};
  a.g = geometry(c);
  const SplitPlan p = plan_splits(c, n, len, bl, a.seqs, ring_extra);
  if (p.max_splits > kvq::kMaxSplits) return fail(KVQ_E_INVALID, "too many splits (%d)", p.max_splits);
  const size_t need = (size_t)n * c->cfg.n_kv_heads * p.max_splits * kPartialFloats(c->cfg.head_dim) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  for (int i = 0; i < n; ++i) a.seqs[i].slab = slab_offset(c, layer, ids[i]);
  a.q = (const uint16_t*)q_bf16;
  a.out = out;
  a.partials = (float*)workspace;
  a.n_seqs = n;
  a.n_q_heads = c->cfg.n_q_heads;
  a.group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  a.max_splits = p.max_splits;
  a.scale = softmax_scale > 0 ? softmax_scale : 1.0f / std::sqrt((float)c->cfg.head_dim);
  hipError_t e = timed(c, KVQ_KERNEL_DECODE, (hipStream_t)stream,
                       [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_decode(a, p.total_wgs, (hipStream_t)stream, e0, e1); });
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  int n_splits[KVQ_MAX_BATCH];
  for (int i = 0; i < n; ++i) n_splits[i] = a.seqs[i].n_body_splits + a.seqs[i].n_ring_splits;
  return launch_combine_for(c, n, n_splits, p.max_splits, out, workspace, (hipStream_t)stream);
}

// ---- multi-query attention (kvq_decode_attn_multi for T >= 2, kvq_prefill_attn): queries in blocks of 16 (two
// per wave) or, with KVarN, a qN_1 body or token-axis K, of 8 (one per wave), each (block, KV head) split so that
// the launch has about one work-group per CU. Without KVarN a split covers any range of the block's tile list (body
// tiles, then ring tiles), so with one split per block the kernel writes the outputs itself; with KVarN the body
// and ring tiles go to separate splits (the body's V values carry sigma_V).

// body length of a sequence after kvq_append of n tokens (the rule kvq_append applies)
int body_len_after(const kvq_cache* c, int layer, int seq, int n) {
  const int k = c->idx(layer, seq);
  if (c->cfg.tail_len == 0) return c->len[k] + n;
  const int over = c->len[k] + n - c->lay.ring_slots;
  if (c->cfg.k_axis) return std::max(c->body_len[k], over > 0 ? (over + kvq::kTile - 1) / kvq::kTile * kvq::kTile : 0);
  return std::max(c->body_len[k], over);
}

long mq_budget(const kvq_cache* c) { return std::min(kDecodeWgsPerCu * c->n_cu, kMaxWgBudget); }

struct MqPlan {
  int total_wgs = 0, max_splits = 1, rows = 0;
  bool partials = false;
};

// Tiles of sequence i's prefix up to position end (body tiles, then ring tiles).
void mq_tiles(int body_len, int end, int& bt, int& rt) {
  bt = (std::min(body_len, end) + kvq::kTile - 1) / kvq::kTile;
  rt = end > body_len ? (end + kvq::kTile - 1) / kvq::kTile - body_len / kvq::kTile : 0;
}

// balance (one block per sequence, kvq_decode_attn_multi): each sequence's splits in proportion to its tiles, at
// most the per-head budget and its tile count (what kvq_workspace_bytes(cache, n_seqs * T, len) provides for);
// otherwise (prefill) every entry the same share, so that rows x splits <= 16 x budget / Hkv
// (kvq_prefill_workspace_bytes).
MqPlan plan_mq(const kvq_cache* c, int n, const int* len, const int* body_len, const int* q0, const int* nq,
               kvq::MqSeq* out, bool balance = false) {
  const int hk = c->cfg.n_kv_heads;
  const int qb = kvq::mq_block_queries(geometry(c));
  long blocks = 0, all_tiles = 0;
  for (int i = 0; i < n; ++i) {
    blocks += (nq[i] + qb - 1) / qb;
    int bt, rt;
    mq_tiles(body_len[i], q0[i] + nq[i], bt, rt);
    all_tiles += bt + rt;
  }
  balance = balance && blocks == n && all_tiles > 0;
  const long entries = std::max(1L, blocks * hk);
  const long budget_h = std::max(1L, mq_budget(c) / hk);
  const int per_entry = (int)std::max(1L, mq_budget(c) / entries);
  MqPlan p;
  for (int i = 0; i < n; ++i) {
    kvq::MqSeq& S = out[i];
    S.len = len[i];
    S.body_len = body_len[i];
    S.q0 = q0[i];
    S.nq = nq[i];
    S.row0 = p.rows;
    int bt, rt;
    mq_tiles(body_len[i], q0[i] + nq[i], bt, rt);
    int ns = std::min(per_entry, std::max(1, bt + rt));
    if (balance)
      ns = (int)std::max(1L, std::min({budget_h * (bt + rt) / all_tiles, budget_h, (long)std::max(1, bt + rt)}));
    int nr = 0;
    if (c->cfg.kvarn && rt > 0) {   // separate body and ring splits
      ns = std::max(ns, bt > 0 ? 2 : 1);
      nr = bt > 0 ? std::max(1, std::min(ns - 1, (int)((long)ns * rt / (bt + rt)))) : ns;
    }
    S.n_splits = ns;
    S.n_ring_splits = nr;
    S.wg_begin = p.total_wgs;
    p.total_wgs += ((nq[i] + qb - 1) / qb) * hk * ns;
    p.max_splits = std::max(p.max_splits, ns);
    p.partials = p.partials || ns > 1;
    p.rows += nq[i];
  }
  return p;
}

size_t mq_partials_bytes(const kvq_cache* c, const MqPlan& p) {
  return p.partials ? (size_t)p.rows * c->cfg.n_kv_heads * p.max_splits * kPartialFloats(c->cfg.head_dim) * sizeof(float)
                    : 0;
}

kvq_status run_mq(kvq_cache* c, int layer, int n, const int32_t* ids, const int* q0, const int* nq, const void* q_bf16,
                  float* out, float softmax_scale, void* workspace, size_t ws_bytes, void* stream,
                  bool balance) {
  kvq::MqArgs a{};
  a.g = geometry(c);
  int len[KVQ_MAX_BATCH], bl[KVQ_MAX_BATCH];
  for (int i = 0; i < n; ++i) {
    const int k = c->idx(layer, ids[i]);
    len[i] = c->len[k];
    bl[i] = c->body_len[k];
  }
  const MqPlan p = plan_mq(c, n, len, bl, q0, nq, a.seqs, balance);
  const size_t need = mq_partials_bytes(c, p);
  if (need && (!workspace || ws_bytes < need)) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  for (int i = 0; i < n; ++i) a.seqs[i].slab = slab_offset(c, layer, ids[i]);
  a.q = (const uint16_t*)q_bf16;
  a.out = out;
  a.partials = (float*)workspace;
  a.n_seqs = n;
  a.n_q_heads = c->cfg.n_q_heads;
  a.group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  a.max_splits = p.max_splits;
  a.scale = softmax_scale > 0 ? softmax_scale : 1.0f / std::sqrt((float)c->cfg.head_dim);
  if (p.total_wgs == 0) return KVQ_OK;
  hipError_t e = timed(c, KVQ_KERNEL_MQ, (hipStream_t)stream,
                       [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_mq(a, p.total_wgs, (hipStream_t)stream, e0, e1); });
  if (e != hipSuccess) return hip_fail(e, "multi-query launch");
  if (p.partials) {
    e = timed(c, KVQ_KERNEL_COMBINE, (hipStream_t)stream,
              [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_mq_combine(a, p.rows, (hipStream_t)stream, e0, e1); });
    if (e != hipSuccess) return hip_fail(e, "multi-query merge launch");
  }
  return KVQ_OK;
}

kvq_status check_decode_args(const void* q_bf16, const float* out, const void* workspace, float softmax_scale) {
  if (!q_bf16 || !out || !workspace) return fail(KVQ_E_INVALID, "q/out/workspace is NULL");
  if (((uintptr_t)workspace) % 256 != 0) return fail(KVQ_E_INVALID, "workspace must be 256-byte aligned");
  if (!std::isfinite(softmax_scale)) return fail(KVQ_E_INVALID, "softmax_scale is not finite");
  return KVQ_OK;
}

}  // namespace
}  // extern "C++"

kvq_status kvq_decode_attn(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q_bf16,
                           float* out, float softmax_scale, void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  s = check_decode_args(q_bf16, out, workspace, softmax_scale);
  if (s != KVQ_OK) return s;
  int len[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) {
    len[i] = c->len[c->idx(layer, seq_ids[i])];
    if (len[i] < 1) return fail(KVQ_E_STATE, "seq %d of layer %d is empty", seq_ids[i], layer);
  }
  return run_decode(c, layer, n_seqs, seq_ids, len, q_bf16, out, softmax_scale, workspace, ws_bytes, stream);
}

kvq_status kvq_decode_attn_noalloc(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                   const void* q_bf16, float* out, float softmax_scale, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (!q_bf16 || !out) return fail(KVQ_E_INVALID, "q/out is NULL");
  if (!std::isfinite(softmax_scale)) return fail(KVQ_E_INVALID, "softmax_scale is not finite");
  int len[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) {
    len[i] = c->len[c->idx(layer, seq_ids[i])];
    if (len[i] < 1) return fail(KVQ_E_STATE, "seq %d of layer %d is empty", seq_ids[i], layer);
  }
  void* scratch = nullptr;
  const hipError_t e = kvq::scratch_device_ptr(c->device, &scratch);
  if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
  s = run_decode(c, layer, n_seqs, seq_ids, len, q_bf16, out, softmax_scale, scratch, kvq::kScratchBytes, stream);
  if (s == KVQ_E_SIZE)
    return fail(KVQ_E_SIZE, "kvq_decode_attn_noalloc: the call's split partials exceed the static scratch of %zu bytes "
                "(%s); use kvq_decode_attn with a workspace", kvq::kScratchBytes, g_err.c_str());
  return s;
}

kvq_status kvq_decode_attn_multi(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                 int32_t n_queries, const void* q_bf16, float* out, float softmax_scale,
                                 void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (n_queries < 1 || n_queries > KVQ_MAX_QUERIES)
    return fail(KVQ_E_INVALID, "n_queries must be in [1, %d] (got %d)", KVQ_MAX_QUERIES, n_queries);
  if (n_seqs * n_queries > KVQ_MAX_BATCH)
    return fail(KVQ_E_INVALID, "n_seqs * n_queries must be at most %d (got %d)", KVQ_MAX_BATCH, n_seqs * n_queries);
  s = check_decode_args(q_bf16, out, workspace, softmax_scale);
  if (s != KVQ_OK) return s;
  int ids[KVQ_MAX_BATCH], len[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) {
    const int n = c->len[c->idx(layer, seq_ids[i])];
    if (n < n_queries)
      return fail(KVQ_E_STATE, "seq %d of layer %d holds %d positions, fewer than %d queries", seq_ids[i], layer, n,
                  n_queries);
    for (int t = 0; t < n_queries; ++t) {   // query t of the sequence sits at position n - n_queries + t
      ids[i * n_queries + t] = seq_ids[i];
      len[i * n_queries + t] = n - n_queries + t + 1;
    }
  }
  if (n_queries > 1 && c->cfg.layout == KVQ_LAYOUT_TILES) {
    // the multi-query kernel: each tile read and decoded once for the T queries of a sequence
    int q0[KVQ_MAX_BATCH], nq[KVQ_MAX_BATCH];
    for (int i = 0; i < n_seqs; ++i) {
      q0[i] = c->len[c->idx(layer, seq_ids[i])] - n_queries;
      nq[i] = n_queries;
    }
    return run_mq(c, layer, n_seqs, seq_ids, q0, nq, q_bf16, out, softmax_scale, workspace, ws_bytes, stream,
                  true);
  }
  // one query per sequence plans (and computes) exactly as kvq_decode_attn; a row-layout cache runs every
  // (sequence, query) pair as an entry of the gather launch
  return run_decode(c, layer, n_seqs * n_queries, ids, len, q_bf16, out, softmax_scale, workspace, ws_bytes, stream,
                    n_queries > 1);
}

size_t kvq_prefill_workspace_bytes(const kvq_cache* c, int32_t n_seqs, int32_t max_new, int32_t max_len) {
  if (!c || n_seqs < 1 || n_seqs > KVQ_MAX_BATCH || max_new < 1 || max_len < 1) return 0;
  // partial records = rows x KV heads x the largest split count. A block holds at most 16 rows and gets at most
  // budget / entries splits (entries >= blocks x Hkv), so rows x splits <= 16 x budget / Hkv; a KVarN block with
  // body and ring tiles takes at least 2 splits; no block takes more splits than its tiles.
  const long rows = (long)n_seqs * std::min(max_new, max_len);
  const long tiles = (max_len + kvq::kTile - 1) / kvq::kTile + 1;
  const long cap = std::max(2L, std::min(tiles, mq_budget(c) / c->cfg.n_kv_heads));
  const long records = std::min(rows * cap, std::max(2 * rows, kvq::kMqBlockPair * mq_budget(c) / c->cfg.n_kv_heads));
  return std::max<size_t>((size_t)records * c->cfg.n_kv_heads * kPartialFloats(c->cfg.head_dim) * sizeof(float), 256);
}

kvq_status kvq_prefill_attn(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                            const void* k_bf16, const void* v_bf16, const void* q_bf16, float* out, float softmax_scale,
                            void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (c->cfg.layout != KVQ_LAYOUT_TILES)
    return fail(KVQ_E_INVALID, "prefill attention reads the tile layout (the cache uses KVQ_LAYOUT_ROWS)");
  if (!n_new) return fail(KVQ_E_INVALID, "n_new is NULL");
  if (!q_bf16 || !out) return fail(KVQ_E_INVALID, "q/out is NULL");
  if (workspace && ((uintptr_t)workspace) % 256 != 0) return fail(KVQ_E_INVALID, "workspace must be 256-byte aligned");
  if (!std::isfinite(softmax_scale)) return fail(KVQ_E_INVALID, "softmax_scale is not finite");
  int q0[KVQ_MAX_BATCH], nq[KVQ_MAX_BATCH], max_new = 0, max_len = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (n_new[i] < 0) return fail(KVQ_E_INVALID, "n_new[%d] is negative", i);
    const int k = c->idx(layer, seq_ids[i]);
    q0[i] = c->len[k];
    nq[i] = n_new[i];
    max_new = std::max(max_new, n_new[i]);
    max_len = std::max(max_len, c->len[k] + n_new[i]);
  }
  if (max_new == 0) return KVQ_OK;
  {   // the workspace this call's plan needs, checked before the append changes anything
    int len[KVQ_MAX_BATCH], bl[KVQ_MAX_BATCH];
    for (int i = 0; i < n_seqs; ++i) {
      len[i] = q0[i] + nq[i];
      bl[i] = body_len_after(c, layer, seq_ids[i], nq[i]);
    }
    kvq::MqSeq seqs[KVQ_MAX_BATCH];
    const size_t need = mq_partials_bytes(c, plan_mq(c, n_seqs, len, bl, q0, nq, seqs));
    if (need && (!workspace || ws_bytes < need))
      return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  }
  s = kvq_append(c, layer, n_seqs, seq_ids, n_new, k_bf16, v_bf16, stream);
  if (s != KVQ_OK) return s;
  return run_mq(c, layer, n_seqs, seq_ids, q0, nq, q_bf16, out, softmax_scale, workspace, ws_bytes, stream);
}

// Tiles the work-group that requantizes a decode step's evicted rows gives up (about the time those writes take).
constexpr int kStepHandicap = 8;

kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* k_bf16,
                           const void* v_bf16, const void* q_bf16, float* out, float softmax_scale, void* workspace,
                           size_t ws_bytes, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  {   // the documented workspace size, checked before anything is appended
    int max_len = 1;
    for (int i = 0; i < n_seqs; ++i) max_len = std::max(max_len, c->len[c->idx(layer, seq_ids[i])] + 1);
    const size_t ws_need = kvq_workspace_bytes(c, n_seqs, max_len);
    if (!workspace || ws_bytes < ws_need) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, ws_need);
  }
  const int W = c->cfg.tail_len;
  const int R = c->lay.ring_slots;
  // One launch when every sequence's step is a ring write plus the requantization of at most the rows of one
  // position tile that were in the ring before the call (the tiles the writes touch then belong to the last
  // ring split and the last body split, which write before they read); otherwise the calls run in turn.
  bool fuse = W > 0 && c->cfg.layout == KVQ_LAYOUT_TILES && !c->cfg.k_min && !c->cfg.v_min && !c->cfg.k_axis &&
              k_bf16 && v_bf16 &&
              q_bf16 && out && workspace &&
              ((uintptr_t)workspace) % 256 == 0 && std::isfinite(softmax_scale);
  int len[KVQ_MAX_BATCH], bl[KVQ_MAX_BATCH], target[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs && fuse; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    len[i] = c->len[k];
    bl[i] = c->body_len[k];
    target[i] = std::max(bl[i], len[i] + 1 - W);
    if ((long)len[i] + 1 > c->cfg.capacity) fuse = false;                 // reported by kvq_append
    else if (c->cfg.kvarn && !c->calibrated[k]) fuse = false;             // calibration comes first
    else if (len[i] + 1 - bl[i] > R) fuse = false;                        // the append would evict itself
    else if (target[i] > len[i]) fuse = false;                            // would evict the new token
    else if (target[i] > bl[i] && bl[i] / kvq::kTile != (target[i] - 1) / kvq::kTile) fuse = false;
  }
  if (!fuse) {
    int32_t ones[KVQ_MAX_BATCH];
    for (int i = 0; i < n_seqs; ++i) ones[i] = 1;
    s = kvq_append_evict(c, layer, n_seqs, seq_ids, ones, k_bf16, v_bf16, stream);
    return s != KVQ_OK ? s : kvq_decode_attn(c, layer, n_seqs, seq_ids, q_bf16, out, softmax_scale, workspace, ws_bytes,
                                              stream);
  }
  int len_new[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) len_new[i] = len[i] + 1;
  kvq::DecodeArgs a{};
  a.g = geometry(c);
  const SplitPlan p = plan_splits(c, n_seqs, len_new, target, a.seqs);
  if (p.max_splits > kvq::kMaxSplits) return fail(KVQ_E_INVALID, "too many splits (%d)", p.max_splits);
  const size_t need = (size_t)n_seqs * c->cfg.n_kv_heads * p.max_splits * kPartialFloats(c->cfg.head_dim) * sizeof(float);
  if (ws_bytes < need) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  for (int i = 0; i < n_seqs; ++i) {
    a.seqs[i].slab = slab_offset(c, layer, seq_ids[i]);
    a.seqs[i].app_pos = len[i];
    a.seqs[i].ev0 = bl[i];
    a.seqs[i].ev1 = target[i];
    // the last body split requantizes the evicted rows before it reads anything: it takes kStepHandicap
    // fewer tiles than an even share (when that leaves it at least one)
    const int nsp = a.seqs[i].n_body_splits;
    const int tiles = (target[i] + kvq::kTile - 1) / kvq::kTile;
    if (target[i] > bl[i] && nsp > 1) {
      const int share = tiles / nsp;
      if (share > kStepHandicap) a.seqs[i].last_tb = tiles - (share - kStepHandicap);
    }
  }
  a.q = (const uint16_t*)q_bf16;
  a.out = out;
  a.partials = (float*)workspace;
  a.k_in = (const uint16_t*)k_bf16;
  a.v_in = (const uint16_t*)v_bf16;
  a.step = 1;
  a.n_seqs = n_seqs;
  a.n_q_heads = c->cfg.n_q_heads;
  a.group = c->cfg.n_q_heads / c->cfg.n_kv_heads;
  a.max_splits = p.max_splits;
  a.scale = softmax_scale > 0 ? softmax_scale : 1.0f / std::sqrt((float)c->cfg.head_dim);
  hipError_t e = timed(c, KVQ_KERNEL_DECODE, (hipStream_t)stream,
                       [&](hipEvent_t e0, hipEvent_t e1) { return kvq::launch_decode(a, p.total_wgs, (hipStream_t)stream, e0, e1); });
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  for (int i = 0; i < n_seqs; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    c->len[k] = len_new[i];
    c->body_len[k] = target[i];
  }
  int n_splits[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) n_splits[i] = a.seqs[i].n_body_splits + a.seqs[i].n_ring_splits;
  return launch_combine_for(c, n_seqs, n_splits, p.max_splits, out, workspace, (hipStream_t)stream);
}

// ------------------------------------------------------------------------------------------ indexer

kvq_status kvq_index_write(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                           const void* key_bf16, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (c->cfg.index_dim == 0) return fail(KVQ_E_INVALID, "the cache has no indexer (index_dim = 0)");
  if (!n_new) return fail(KVQ_E_INVALID, "n_new is NULL");
  kvq::IndexWriteArgs a{};
  a.g = geometry(c);
  a.key_in = (const uint16_t*)key_bf16;
  a.pool = c->cfg.index_pool;
  int total = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int len = c->len[c->idx(layer, seq_ids[i])];
    if (n_new[i] < 0) return fail(KVQ_E_INVALID, "n_new[%d] is negative", i);
    if (n_new[i] > len)
      return fail(KVQ_E_STATE, "seq %d holds %d positions, fewer than %d index keys", seq_ids[i], len, n_new[i]);
    if (n_new[i] == 0) continue;
    a.items[a.n_items++] = kvq::IndexWriteItem{slab_offset(c, layer, seq_ids[i]), len - n_new[i], n_new[i], total, total};
    total += n_new[i];
  }
  if (total == 0) return KVQ_OK;
  if (!key_bf16) return fail(KVQ_E_INVALID, "key input is NULL");
  hipError_t e = timed(c, KVQ_KERNEL_APPEND, (hipStream_t)stream, [&](hipEvent_t e0, hipEvent_t e1) {
    return kvq::launch_index_write(a, total, (hipStream_t)stream, e0, e1);
  });
  if (e != hipSuccess) return hip_fail(e, "index write launch");
  return KVQ_OK;
}

extern "C++" {
namespace {
int index_wgs(int m) { return std::max(1, (m + kvq::kIndexChunk - 1) / kvq::kIndexChunk); }
}  // namespace
}  // extern "C++"

size_t kvq_index_workspace_bytes(const kvq_cache* c, int32_t n_seqs, int32_t max_len) {
  if (!c || n_seqs < 1 || max_len < 0) return 0;
  return (size_t)n_seqs * kvq::index_ws_seq_bytes(index_wgs(max_len));
}

kvq_status kvq_index_select(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const void* query_bf16, int32_t budget, int32_t n_recent, int32_t* positions,
                            void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (c->cfg.index_dim == 0) return fail(KVQ_E_INVALID, "the cache has no indexer (index_dim = 0)");
  if (!query_bf16 || !positions || !workspace) return fail(KVQ_E_INVALID, "query/positions/workspace is NULL");
  if (((uintptr_t)workspace) % 256 != 0) return fail(KVQ_E_INVALID, "workspace must be 256-byte aligned");
  if (((uintptr_t)positions) % 4 != 0) return fail(KVQ_E_INVALID, "positions must be 4-byte aligned");
  if (budget < 1 || budget > (1 << 28)) return fail(KVQ_E_INVALID, "budget must be in [1, 2^28] (got %d)", budget);
  if (n_recent < 0 || n_recent > budget)
    return fail(KVQ_E_INVALID, "n_recent must be in [0, budget] (got %d, budget %d)", n_recent, budget);
  kvq::IndexArgs a{};
  a.g = geometry(c);
  a.q = (const uint16_t*)query_bf16;
  a.out = positions;
  a.ws = (uint8_t*)workspace;
  a.budget = budget;
  a.n_seqs = n_seqs;
  size_t off = 0;
  int wgs = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int len = c->len[c->idx(layer, seq_ids[i])];
    const int recent = std::min(n_recent, len);
    kvq::IndexSeq& S = a.seqs[i];
    S.slab = slab_offset(c, layer, seq_ids[i]);
    S.ws_off = off;
    S.len = len;
    S.m = len - recent;
    S.k = budget - recent;
    S.n_wgs = index_wgs(S.m);
    S.wg_begin = wgs;
    wgs += S.n_wgs;
    off += kvq::index_ws_seq_bytes(S.n_wgs);
  }
  if (ws_bytes < off) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, off);
  hipError_t e = timed(c, KVQ_KERNEL_INDEX, (hipStream_t)stream, [&](hipEvent_t e0, hipEvent_t e1) {
    return kvq::launch_index_select(a, wgs, (hipStream_t)stream, e0, e1);
  });
  if (e != hipSuccess) return hip_fail(e, "index select launch");
  return KVQ_OK;
}

// Host checks of a sparse decode call (before any work).
static kvq_status check_sparse(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids, const void* q_bf16,
                               const int32_t* positions, int32_t budget, const float* out, float softmax_scale,
                               const void* workspace) {
  kvq_status s = check_seqs(c, layer, n_seqs, seq_ids);
  if (s != KVQ_OK) return s;
  if (c->cfg.layout != KVQ_LAYOUT_ROWS)
    return fail(KVQ_E_INVALID, "sparse decode reads whole rows: the cache must use KVQ_LAYOUT_ROWS");
  if (!q_bf16 || !out || !workspace || !positions) return fail(KVQ_E_INVALID, "q/positions/out/workspace is NULL");
  if (((uintptr_t)workspace) % 256 != 0) return fail(KVQ_E_INVALID, "workspace must be 256-byte aligned");
  if (((uintptr_t)positions) % 4 != 0) return fail(KVQ_E_INVALID, "positions must be 4-byte aligned");
  if (budget < 1 || budget > (1 << 28)) return fail(KVQ_E_INVALID, "budget must be in [1, 2^28] (got %d)", budget);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_E_INVALID, "softmax_scale is not finite");
  return KVQ_OK;
}

kvq_status kvq_sparse_decode_attn(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                  const void* q_bf16, const int32_t* positions, int32_t budget, float* out,
                                  float softmax_scale, void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_sparse(c, layer, n_seqs, seq_ids, q_bf16, positions, budget, out, softmax_scale, workspace);
  if (s != KVQ_OK) return s;
  int n_list[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) n_list[i] = budget;
  return run_gather(c, layer, n_seqs, seq_ids, q_bf16, positions, budget, n_list, out, softmax_scale, workspace,
                    ws_bytes, stream);
}

kvq_status kvq_sparse_decode_step(kvq_cache* c, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                  const void* k_bf16, const void* v_bf16, const void* q_bf16,
                                  const int32_t* positions, int32_t budget, float* out, float softmax_scale,
                                  void* workspace, size_t ws_bytes, void* stream) {
  kvq_status s = check_sparse(c, layer, n_seqs, seq_ids, q_bf16, positions, budget, out, softmax_scale, workspace);
  if (s != KVQ_OK) return s;
  // the documented workspace size, checked before anything is appended
  const size_t ws_need = kvq_workspace_bytes(c, n_seqs, budget);
  if (ws_bytes < ws_need) return fail(KVQ_E_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, ws_need);
  // one launch when the new rows go straight to the body (no ring) and are quantized with known scales
  bool fuse = c->cfg.tail_len == 0 && k_bf16 && v_bf16;
  for (int i = 0; i < n_seqs && fuse; ++i) {
    const int k = c->idx(layer, seq_ids[i]);
    if ((long)c->len[k] + 1 > c->cfg.capacity) fuse = false;               // reported by kvq_append
    else if (c->cfg.kvarn && !c->calibrated[k]) fuse = false;             // calibration comes first
  }
  if (!fuse) {
    int32_t ones[KVQ_MAX_BATCH];
    for (int i = 0; i < n_seqs; ++i) ones[i] = 1;
    s = kvq_append(c, layer, n_seqs, seq_ids, ones, k_bf16, v_bf16, stream);
    return s != KVQ_OK ? s : kvq_sparse_decode_attn(c, layer, n_seqs, seq_ids, q_bf16, positions, budget, out,
                                                     softmax_scale, workspace, ws_bytes, stream);
  }
  int n_list[KVQ_MAX_BATCH];
  for (int i = 0; i < n_seqs; ++i) n_list[i] = budget;
  return run_gather(c, layer, n_seqs, seq_ids, q_bf16, positions, budget, n_list, out, softmax_scale, workspace,
                    ws_bytes, stream, k_bf16, v_bf16);
}

}  // extern "C"
