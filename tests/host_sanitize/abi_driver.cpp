// Host-only exercise of the kvq C ABI for a build under AddressSanitizer and UndefinedBehaviorSanitizer: kernel
// launches are stubs (launch_stubs.cpp) and the "device" pointers are never dereferenced by the host code, so
// the run covers validation, size and region arithmetic, split and block planning, workspace checks and every
// error return on a machine without a GPU. Exits 0 when every checked status is the expected one.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvq.h"

extern "C" long kvq_stub_launches();

namespace {
int g_fail = 0;
void expect(kvq_status got, kvq_status want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, (int)got, (int)want, kvq_last_error());
    ++g_fail;
  }
}
void in_range(kvq_status got, const char* what, int line) {
  if ((int)got > 0 || (int)got < -5) {
    std::fprintf(stderr, "line %d: %s returned %d, not a kvq_status\n", line, what, (int)got);
    ++g_fail;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)
#define ANY(call) in_range((call), #call, __LINE__)

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
int rnd(int lo, int hi) {   // inclusive range, xorshift64
  g_rng ^= g_rng << 13; g_rng ^= g_rng >> 7; g_rng ^= g_rng << 17;
  return lo + (int)(g_rng % (uint64_t)(hi - lo + 1));
}

// Fake device addresses: 256-byte aligned, never dereferenced on the host.
void* fake(uint64_t k) { return (void*)(uintptr_t)(0x100000000000ull + (k << 28)); }

kvq_config base() {
  kvq_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 2; c.max_seqs = 4; c.capacity = 5000; c.n_q_heads = 16; c.n_kv_heads = 2; c.head_dim = 256;
  c.k_bits = 6; c.v_bits = 5; c.tail_len = 128; c.tail_slack = 32; c.tail_dtype = KVQ_TAIL_BF16;
  return c;
}

void random_configs() {
  for (int it = 0; it < 4000; ++it) {
    kvq_config c = base();
    c.n_layers = rnd(-1, 40); c.max_seqs = rnd(-1, 70); c.capacity = rnd(-5, 1 << 20);
    c.n_kv_heads = rnd(0, 9); c.n_q_heads = c.n_kv_heads * rnd(0, 9) + (rnd(0, 7) == 0);
    c.head_dim = rnd(0, 3) ? 256 : rnd(0, 512);
    c.k_bits = rnd(1, 9); c.v_bits = rnd(1, 9); c.kvarn = rnd(-1, 2);
    c.tail_len = rnd(0, 3) ? 32 * rnd(0, 70) : rnd(-3, 3000); c.tail_slack = 32 * rnd(-1, 20);
    c.tail_dtype = rnd(-1, 4); c.layout = rnd(-1, 2);
    const int pool = rnd(0, 5) ? 1 << rnd(0, 4) : rnd(-1, 40);
    c.index_pool = pool; c.index_dim = rnd(0, 1) ? 32 * pool : rnd(0, 300) * rnd(0, 1);
    c.k_min = rnd(-1, 2) == 1; c.v_min = rnd(0, 2) == 1; c.k_axis = rnd(0, 3) == 1;
    const kvq_status v = kvq_config_validate(&c);
    in_range(v, "kvq_config_validate", __LINE__);
    const size_t bytes = kvq_cache_bytes(&c);
    if ((v == KVQ_OK) != (bytes > 0)) {
      std::fprintf(stderr, "config %d: validate %d but cache_bytes %zu\n", it, (int)v, bytes);
      ++g_fail;
    }
    if (v != KVQ_OK) continue;
    size_t prev_end = 0;
    for (int l = 0; l < c.n_layers; l += (c.n_layers > 3 ? c.n_layers - 1 : 1))
      for (int s = 0; s < c.max_seqs; s += (c.max_seqs > 3 ? c.max_seqs - 1 : 1)) {
        size_t off = 0, sz = 0;
        EXPECT(kvq_region(&c, l, s, KVQ_REGION_SLAB, &off, &sz), KVQ_OK);
        if (off + sz > bytes || off < prev_end) { std::fprintf(stderr, "slab %d/%d outside the arena\n", l, s); ++g_fail; }
        prev_end = off + sz;
        for (int r = 0; r <= KVQ_REGION_INDEX; ++r) ANY(kvq_region(&c, l, s, r, &off, &sz));
      }
    size_t off, sz;
    EXPECT(kvq_region(&c, c.n_layers, 0, KVQ_REGION_SLAB, &off, &sz), KVQ_E_INVALID);
    EXPECT(kvq_region(&c, 0, c.max_seqs, KVQ_REGION_SLAB, &off, &sz), KVQ_E_INVALID);
    EXPECT(kvq_region(&c, 0, 0, 99, &off, &sz), KVQ_E_INVALID);
    EXPECT(kvq_region(&c, 0, 0, KVQ_REGION_SLAB, nullptr, &sz), KVQ_E_INVALID);
  }
}

void null_arguments() {
  EXPECT(kvq_config_validate(nullptr), KVQ_E_INVALID);
  if (kvq_cache_bytes(nullptr) != 0) ++g_fail;
  kvq_config c = base();
  kvq_cache* h = nullptr;
  EXPECT(kvq_cache_init(&c, fake(1), kvq_cache_bytes(&c), nullptr, nullptr), KVQ_E_INVALID);
  EXPECT(kvq_cache_init(&c, nullptr, kvq_cache_bytes(&c), nullptr, &h), KVQ_E_INVALID);
  EXPECT(kvq_cache_init(&c, (char*)fake(1) + 16, kvq_cache_bytes(&c), nullptr, &h), KVQ_E_INVALID);
  EXPECT(kvq_cache_init(&c, fake(1), kvq_cache_bytes(&c) - 1, nullptr, &h), KVQ_E_SIZE);
  const int32_t id = 0, one = 1;
  EXPECT(kvq_append(nullptr, 0, 1, &id, &one, fake(2), fake(3), nullptr), KVQ_E_INVALID);
  EXPECT(kvq_tail_evict(nullptr, 0, 1, &id, nullptr), KVQ_E_INVALID);
  EXPECT(kvq_decode_attn(nullptr, 0, 1, &id, fake(4), (float*)fake(5), 0.f, fake(6), 1 << 20, nullptr), KVQ_E_INVALID);
  EXPECT(kvq_seq_lengths(nullptr, 0, 0, nullptr, nullptr), KVQ_E_INVALID);
  if (kvq_workspace_bytes(nullptr, 1, 1) != 0) ++g_fail;
  kvq_cache_destroy(nullptr);
  if (!kvq_last_error()) ++g_fail;
}

// A scripted sequence of calls on one cache; the statuses of the valid calls must be KVQ_OK.
void session(kvq_config c, bool sparse_layer) {
  const size_t bytes = kvq_cache_bytes(&c);
  kvq_cache* h = nullptr;
  EXPECT(kvq_cache_init(&c, fake(1), bytes, nullptr, &h), KVQ_OK);
  if (!h) return;
  const int n = c.max_seqs < 3 ? c.max_seqs : 3;
  std::vector<int32_t> ids(n), n_new(n), lens(n);
  for (int i = 0; i < n; ++i) ids[i] = c.max_seqs - 1 - i;
  void *k = fake(2), *v = fake(3), *q = fake(4), *ws = fake(6), *key = fake(7);
  float* out = (float*)fake(5);
  int32_t* pos = (int32_t*)fake(8);
  for (int layer = 0; layer < c.n_layers; ++layer) {
    for (int chunk = 0; chunk < 3; ++chunk) {
      for (int i = 0; i < n; ++i) n_new[i] = chunk == 1 && i == 0 ? 0 : rnd(1, c.capacity / 8);
      EXPECT(kvq_append(h, layer, n, ids.data(), n_new.data(), k, v, nullptr), KVQ_OK);
      if (c.index_dim) EXPECT(kvq_index_write(h, layer, n, ids.data(), n_new.data(), key, nullptr), KVQ_OK);
    }
    if (c.tail_len) EXPECT(kvq_tail_evict(h, layer, n, ids.data(), nullptr), KVQ_OK);
    int max_len = 1;
    for (int i = 0; i < n; ++i) {
      int32_t bl = 0;
      EXPECT(kvq_seq_lengths(h, layer, ids[i], &lens[i], &bl), KVQ_OK);
      if (bl > lens[i]) ++g_fail;
      max_len = lens[i] + 16 > max_len ? lens[i] + 16 : max_len;
    }
    const size_t wsb = kvq_workspace_bytes(h, n * 8, max_len);
    if (wsb == 0) ++g_fail;
    EXPECT(kvq_decode_attn(h, layer, n, ids.data(), q, out, 0.f, ws, wsb, nullptr), KVQ_OK);
    EXPECT(kvq_decode_attn(h, layer, n, ids.data(), q, out, 0.f, ws, 16, nullptr), KVQ_E_SIZE);
    ANY(kvq_decode_attn_noalloc(h, layer, n, ids.data(), q, out, 0.f, nullptr));
    for (int s = 0; s < 4; ++s) {
      std::vector<int32_t> ones(n, 1);
      EXPECT(kvq_decode_step(h, layer, n, ids.data(), k, v, q, out, 0.f, ws, wsb, nullptr), KVQ_OK);
      EXPECT(kvq_append_evict(h, layer, n, ids.data(), ones.data(), k, v, nullptr), KVQ_OK);
    }
    for (int T = 1; T <= KVQ_MAX_QUERIES; ++T) ANY(kvq_decode_attn_multi(h, layer, n, ids.data(), T, q, out, 0.f, ws, wsb, nullptr));
    EXPECT(kvq_decode_attn_multi(h, layer, n, ids.data(), KVQ_MAX_QUERIES + 1, q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    {
      std::vector<int32_t> nl(n);
      for (int i = 0; i < n; ++i) { int32_t bl; kvq_seq_lengths(h, layer, ids[i], &nl[i], &bl); nl[i] = nl[i] - 1 > bl ? nl[i] - 1 : bl; }
      ANY(kvq_seq_truncate(h, layer, n, ids.data(), nl.data()));
      for (int i = 0; i < n; ++i) nl[i] = -1;
      EXPECT(kvq_seq_truncate(h, layer, n, ids.data(), nl.data()), KVQ_E_INVALID);
    }
    {
      std::vector<int32_t> pn(n);
      for (int i = 0; i < n; ++i) pn[i] = rnd(0, 300);
      const size_t pws = kvq_prefill_workspace_bytes(h, n, 300, max_len + 300);
      ANY(kvq_prefill_attn(h, layer, n, ids.data(), pn.data(), k, v, q, out, 0.f, ws, pws, nullptr));
      // (prefill reads the tile layout: a row-layout cache refuses it before the workspace check)
      EXPECT(kvq_prefill_attn(h, layer, n, ids.data(), pn.data(), k, v, q, out, 0.f, ws, 0, nullptr),
             sparse_layer ? KVQ_E_INVALID : KVQ_E_SIZE);
    }
    const int budget = rnd(1, 2048);
    if (sparse_layer) {
      EXPECT(kvq_sparse_decode_attn(h, layer, n, ids.data(), q, pos, budget, out, 0.f, ws, wsb, nullptr), KVQ_OK);
      ANY(kvq_sparse_decode_step(h, layer, n, ids.data(), k, v, q, pos, budget, out, 0.f, ws, wsb, nullptr));
    } else {
      ANY(kvq_sparse_decode_attn(h, layer, n, ids.data(), q, pos, budget, out, 0.f, ws, wsb, nullptr));
    }
    if (c.index_dim) {
      const size_t iws = kvq_index_workspace_bytes(h, n, max_len + 64);
      EXPECT(kvq_index_select(h, layer, n, ids.data(), q, budget, budget / 4, pos, ws, iws, nullptr), KVQ_OK);
      EXPECT(kvq_index_select(h, layer, n, ids.data(), q, budget, budget + 1, pos, ws, iws, nullptr), KVQ_E_INVALID);
    }
    // invalid sequence lists and layers
    std::vector<int32_t> dup(2, ids[0]);
    EXPECT(kvq_decode_attn(h, layer, 2, dup.data(), q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    int32_t bad = c.max_seqs;
    EXPECT(kvq_decode_attn(h, layer, 1, &bad, q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    EXPECT(kvq_decode_attn(h, c.n_layers, n, ids.data(), q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    EXPECT(kvq_decode_attn(h, layer, 0, ids.data(), q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    EXPECT(kvq_decode_attn(h, layer, KVQ_MAX_BATCH + 1, ids.data(), q, out, 0.f, ws, wsb, nullptr), KVQ_E_INVALID);
    // past the capacity
    std::vector<int32_t> big(n, c.capacity);
    EXPECT(kvq_append(h, layer, n, ids.data(), big.data(), k, v, nullptr), KVQ_E_CAPACITY);
  }
  EXPECT(kvq_seq_reset(h, -1, n, ids.data(), nullptr), KVQ_OK);
  int32_t len = -1, bl = -1;
  EXPECT(kvq_seq_lengths(h, 0, ids[0], &len, &bl), KVQ_OK);
  if (len != 0 || bl != 0) ++g_fail;
  double ms = 0;
  int32_t launches = 0;
  ANY(kvq_timing_read(h, KVQ_KERNEL_DECODE, &ms, &launches));
  EXPECT(kvq_timing_read(h, 99, &ms, &launches), KVQ_E_INVALID);
  kvq_cache_destroy(h);
}
}  // namespace

int main() {
  random_configs();
  null_arguments();
  kvq_config c = base();
  session(c, false);                                              // K6/V5 + bf16 tail
  c.tail_dtype = KVQ_TAIL_Q8_0; session(c, false);                // 8-bit ring
  c.tail_dtype = KVQ_TAIL_F16; c.kvarn = 1; c.k_bits = 4; c.v_bits = 4; session(c, false);
  c = base(); c.tail_len = 0; c.tail_slack = 0; c.k_bits = 8; c.v_bits = 8; c.layout = KVQ_LAYOUT_ROWS;
  c.index_dim = 128; c.index_pool = 4; session(c, true);          // sparse layer with an indexer
  c = base(); c.k_min = 1; c.v_min = 1; session(c, false);        // qN_1 bodies
  c = base(); c.k_axis = 1; c.tail_slack = 64; session(c, false); // token-axis K
  c = base(); c.max_seqs = 1; c.n_kv_heads = 1; c.n_q_heads = 8; c.capacity = 300; c.tail_len = 32; session(c, false);
  std::printf("abi_driver: %d failed checks, %ld stub launches\n", g_fail, kvq_stub_launches());
  return g_fail ? 1 : 0;
}
