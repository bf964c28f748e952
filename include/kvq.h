/*
 * kvq — mixed-precision quantized KV cache and the decode attention that reads it (MI355X / gfx950).
 *
 * C ABI. Every entry point takes plain pointers and sizes; device pointers are HIP device memory owned
 * by the caller, host pointers are ordinary host memory read during the call only. Nothing here
 * allocates device memory. All GPU work is enqueued asynchronously on the caller's stream (a
 * hipStream_t passed as void*; NULL = the default stream). Calls on one cache handle must be ordered
 * on one stream; a handle is not thread-safe.
 *
 * Errors: every call validates its arguments and the cache state on the host before any HIP call and
 * returns a kvq_status; no exception crosses the ABI. A launch failure returns KVQ_E_HIP. A fault
 * inside a kernel surfaces at the caller's next stream synchronisation. kvq_last_error() returns a
 * thread-local message describing the last failure.
 *
 * Passages cited: "BeeLlama.cpp v0.4.1" page (KV cache types q2_0..q8_0, KVarN, precision tail);
 * "KV cache quant benchmarks: KVarN 6-bit matches q8_0, 4-bit matches q5_0" page (separate K and V
 * types, cache-size column); "Hard numbers on Qwen3.8-27B's KV cache" page (K 6-bit / V 5-bit with a
 * 2,048-position 8-bit ring; requantization when the window moves); "You can offload most of
 * Qwen3.8-Flash-Next's KV cache to RAM" page (decode reads the whole cache of a full-attention layer;
 * a QSA layer reads only an indexer-chosen budget of positions).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_E_INVALID = -1,   /* bad argument or configuration                                   */
  KVQ_E_CAPACITY = -2,  /* an append would exceed the per-sequence capacity                 */
  KVQ_E_SIZE = -3,      /* a caller buffer (arena, workspace) is too small                  */
  KVQ_E_HIP = -4,       /* a HIP runtime call or kernel launch failed                        */
  KVQ_E_STATE = -5      /* the call is not valid in the cache's current state (e.g. empty)   */
} kvq_status;

typedef enum {
  KVQ_TAIL_NONE = 0,    /* no precision tail: every token goes straight to the qN_0 body          */
  KVQ_TAIL_BF16 = 1,    /* newest tail_len tokens kept in bf16 (BeeLlama page, precision tail)     */
  KVQ_TAIL_Q8_0 = 2,    /* newest tail_len tokens kept as q8_0 (Qwen3.8-27B page, 8-bit ring)      */
  KVQ_TAIL_F16 = 3      /* newest tail_len tokens kept in f16 (BeeLlama page, precision tail: BF16 or
                         * F16): the bf16 input rounded to IEEE binary16, nearest even; magnitudes
                         * above 65504 become infinite (the caller keeps K, V in f16 range)       */
} kvq_tail_dtype;

typedef enum {
  KVQ_LAYOUT_TILES = 0, /* V (and q8_0 ring V) stored in 32-position tiles ordered for the decode kernel's
                           matrix operands: the fastest dense decode; no sparse decode              */
  KVQ_LAYOUT_ROWS = 1   /* every K and V position stored as one row, position-major: a position's K and V
                           rows of all KV heads are one contiguous run (the K body / K ring regions hold
                           them; the V regions are empty), so that a sparse layer gathers exactly the rows
                           it attends in whole runs (offload page, QSA paragraph)                     */
} kvq_layout;

/* Maximum number of sequences one call may name. */
#define KVQ_MAX_BATCH 64

/* Maximum queries per sequence of kvq_decode_attn_multi: the token being verified plus up to 7 drafts. */
#define KVQ_MAX_QUERIES 8

/* Cache configuration. K and V bit widths are chosen separately (KVarN benchmark page, K/V pairs). */
typedef struct {
  int32_t n_layers;     /* layers held by the arena                                        */
  int32_t max_seqs;     /* sequence slots per layer; sequence ids are 0..max_seqs-1          */
  int32_t capacity;     /* maximum positions per sequence                                    */
  int32_t n_q_heads;    /* query heads; n_q_heads / n_kv_heads <= 8                           */
  int32_t n_kv_heads;   /* KV heads                                                          */
  int32_t head_dim;     /* 256 (the layout also covers 128; kernels are built for 256)       */
  int32_t k_bits;       /* 2..8: code width of the K body (qN_0, or qN_1 with k_min)           */
  int32_t v_bits;       /* 2..8: code width of the V body (qN_0, or qN_1 with v_min)           */
  int32_t kvarn;        /* 0/1: per-channel variance normalization before block quantization */
  int32_t tail_len;     /* W: newest tokens kept in the tail ring (0 = no ring)                */
  int32_t tail_slack;   /* S: extra ring slots; ring capacity R = W + S must be a multiple of 32 */
  int32_t tail_dtype;   /* kvq_tail_dtype (ignored when tail_len == 0)                          */
  int32_t layout;       /* kvq_layout: placement of V rows (both layouts have the same size)       */
  int32_t index_dim;    /* 0: no indexer; else the QSA indexer head dim, whose keys are pooled to 32 values
                           (offload page: indexer_head_dim 128, compress ratio 4): index_dim = 32 x index_pool */
  int32_t index_pool;   /* pooling ratio of the index keys: 1, 2, 4, 8 or 16 (ignored when index_dim == 0)  */
  int32_t k_min;        /* 0: K body qN_0 (one fp16 scale per 32 values); 1: qN_1, a scale and an fp16 minimum
                           per 32 values, value = scale x code + minimum with codes 0..2^N-1 (BeeLlama page,
                           q2_1 .. q6_1; KVarN benchmark page, q5_1 and q8_0-q5_1). Needs KVQ_LAYOUT_TILES.   */
  int32_t v_min;        /* 0/1: the same for the V body                                                    */
  int32_t k_axis;       /* 0: a K block is 32 channels of one position; 1: token axis, a K block is the 32
                           positions of one channel in a position tile (KIVI-style per-channel K, Qwen3.8-27B
                           page, reader comment). A tile's K is quantized once all its positions are known, so
                           the body grows by whole tiles and the ring holds the window plus the tile still
                           filling: needs KVQ_LAYOUT_TILES, tail_len >= 1 and tail_slack >= 32; kvq_tail_evict
                           then keeps between tail_len and tail_len + 31 positions in the ring.            */
} kvq_config;

typedef struct kvq_cache kvq_cache;

/* Regions of one (layer, sequence) slab, for kvq_region(). */
enum { KVQ_REGION_K_BODY = 0, KVQ_REGION_V_BODY = 1, KVQ_REGION_K_RING = 2, KVQ_REGION_V_RING = 3,
       KVQ_REGION_SIGMA = 4, KVQ_REGION_SLAB = 5, KVQ_REGION_INDEX = 6 };

/* Validate a configuration (host only). */
kvq_status kvq_config_validate(const kvq_config* cfg);

/* Exact arena size in bytes for cfg (0 if cfg is invalid). The body costs N bits per value plus one
 * fp16 scale (qN_1: and one fp16 minimum) per 32 values; a tail ring costs R slots of bf16 or q8_0 rows; KVarN adds D fp16 scales
 * per (layer, sequence, KV head, K/V). At 16 layers x 4 KV heads x 256 x 65,536 positions this gives the
 * BeeLlama page's KV MiB column for q4_0..q8_0 at tail 0 / 1024 / 2048. */
size_t kvq_cache_bytes(const kvq_config* cfg);

/* Byte offset and size of a region of the (layer, seq) slab inside the arena (host only). */
kvq_status kvq_region(const kvq_config* cfg, int32_t layer, int32_t seq, int32_t region,
                      size_t* offset, size_t* bytes);

/* Create a host handle over a caller-owned device arena of at least kvq_cache_bytes(cfg) bytes
 * (256-byte aligned). The arena is zero-filled on `stream`; every sequence starts empty. The handle
 * records the arena pointer, the configuration and per-(layer, sequence) lengths; it owns no device
 * memory. */
kvq_status kvq_cache_init(const kvq_config* cfg, void* dev_arena, size_t arena_bytes, void* stream,
                          kvq_cache** out);

/* Free the host handle (the arena stays the caller's). */
void kvq_cache_destroy(kvq_cache* cache);

/* Forget the contents of sequences (lengths and KVarN calibration back to zero) and zero their slabs
 * for the given layer (layer = -1: every layer). seq_ids: host int32[n_seqs]. */
kvq_status kvq_seq_reset(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                         void* stream);

/* Drop the newest positions of each listed sequence of a layer down to new_len[i] (host int32[n_seqs]), as
 * after a verification step that rejected drafted tokens (Qwen3.8-27B page, decode-speed paragraph on MTP
 * drafting): only rows still in the ring can be dropped, so body_len <= new_len[i] <= len (keep drafts in the
 * ring: tail_len at least the number of drafts, and evict after the verification, not before). The dropped ring
 * rows need no clearing (later appends write their slots again); KVarN calibration is kept. Host state only:
 * ordered before every later launch on any stream.
 * Errors: KVQ_E_INVALID if new_len[i] is outside [0, len]; KVQ_E_STATE if it is below body_len. No sequence is
 * changed when an error is returned. */
kvq_status kvq_seq_truncate(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const int32_t* new_len);

/* Host-side lengths of a (layer, seq): positions held (len) and positions in the qN_0 body. */
kvq_status kvq_seq_lengths(const kvq_cache* cache, int32_t layer, int32_t seq, int32_t* len,
                           int32_t* body_len);

/* Workspace bytes needed by kvq_decode_attn / kvq_sparse_decode_attn for n_seqs sequences of at most
 * max_len positions (sparse: max_len = budget). */
size_t kvq_workspace_bytes(const kvq_cache* cache, int32_t n_seqs, int32_t max_len);

/* Append n_new[i] tokens to sequence seq_ids[i] of `layer`.
 * seq_ids, n_new: host int32[n_seqs] (distinct ids). k_bf16, v_bf16: device bf16 [sum n_new][Hkv][D],
 * sequences packed in call order. The first non-empty append of a (layer, seq) calibrates the KVarN
 * scales from its tokens (BeeLlama page, KVarN). With a tail ring the new tokens enter the ring; when
 * the ring (R = W + S slots) would overflow, its oldest rows are first requantized into the body
 * (Qwen3.8-27B page, window boundary), and new tokens already behind the window go to the body through
 * the ring representation, so the body never depends on how tokens were chunked. Without a ring tokens
 * are quantized straight into the body. Errors: KVQ_E_CAPACITY if len + n_new > capacity. */
kvq_status kvq_append(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                      const int32_t* n_new, const void* k_bf16, const void* v_bf16, void* stream);

/* Requantize ring rows older than the newest tail_len into the body (Qwen3.8-27B page: blocks are
 * requantized when the window boundary moves). After the call the ring holds exactly the newest
 * min(len, W) positions. No-op without a ring. seq_ids: host int32[n_seqs]. */
kvq_status kvq_tail_evict(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                          void* stream);

/* kvq_append followed by kvq_tail_evict on the same sequences, with the same result. When every sequence's
 * evicted positions were already in the ring before the call and the new tokens fit the ring beside them
 * (a decode step: append one token, requantize the one leaving the window), both run in a single kernel
 * launch; otherwise the two calls run in turn. Arguments and errors as kvq_append. */
kvq_status kvq_append_evict(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const int32_t* n_new, const void* k_bf16, const void* v_bf16, void* stream);

/* Dense decode attention (offload page: each step reads the whole cache of a full-attention
 * layer). With KVQ_LAYOUT_ROWS the rows are read by the same gather kernel as sparse decode. For each sequence i: out[i][h][:] = softmax(scale * q[i][h] . K^[t]) over t in [0, len) of V^,
 * with K^, V^ the dequantized body rows (t < body_len) or ring rows. q_bf16: device bf16
 * [n_seqs][Hq][D]; out: device fp32 [n_seqs][Hq][D]; softmax_scale <= 0 means 1/sqrt(D); workspace:
 * device, at least kvq_workspace_bytes(cache, n_seqs, max len) bytes, 256-byte aligned, no initial
 * contents needed. Work-groups over (position split, KV head, sequence) write partial (max, sum, output)
 * records to the workspace; a second kernel merges them with a log-sum-exp. Calls that may run
 * concurrently must not share a workspace.
 * Errors: KVQ_E_STATE if a sequence is empty; KVQ_E_SIZE if the workspace is too small. */
kvq_status kvq_decode_attn(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                           const void* q_bf16, float* out, float softmax_scale, void* workspace,
                           size_t ws_bytes, void* stream);

/* kvq_decode_attn without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The split partials go to the
 * library's static scratch: 16 MiB of device memory per GPU, held from the first kvq_cache_init on that GPU
 * until the process ends; results are those of kvq_decode_attn. Every call on one GPU uses the same scratch,
 * so calls that may overlap on one GPU (other streams, other threads, other caches) race and must be
 * serialized by the caller; the scratch needs no initial contents (each call writes every partial it reads).
 * Arguments and errors as kvq_decode_attn; KVQ_E_SIZE if the call's partials exceed the scratch: they take
 * n_seqs x n_kv_heads x (the most splits planned for one of the sequences) records of 8 x (head_dim + 2) fp32,
 * at most 2,032 records at head_dim 256 (one sequence of any length fits; a call for which
 * kvq_workspace_bytes(cache, n_seqs, max len) <= 16 MiB always fits). */
kvq_status kvq_decode_attn_noalloc(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                   const void* q_bf16, float* out, float softmax_scale, void* stream);

/* One decode step of every listed sequence: append one token each (k_bf16, v_bf16: device bf16
 * [n_seqs][Hkv][D]) and requantize the ring rows that leave the window, then dense decode attention, with
 * the results of kvq_append_evict (n_new = 1 each) followed by kvq_decode_attn. With the tile layout and a
 * ring, when the step is a ring write plus the requantization of rows that were in the ring before the call
 * (every step after the prefill), the writes are done inside the decode launch by the work-groups that read
 * those tiles, before they read them; otherwise the calls run in turn. Arguments and errors as those calls;
 * the workspace size (kvq_workspace_bytes for the lengths after the append) is checked before any write. */
kvq_status kvq_decode_step(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                           const void* k_bf16, const void* v_bf16, const void* q_bf16, float* out,
                           float softmax_scale, void* workspace, size_t ws_bytes, void* stream);

/* Dense decode of T = n_queries queries per sequence in one call, as when the last accepted token and up
 * to 7 drafted ones are verified together (Qwen3.8-27B page, decode-speed paragraph: the engine drafts up to
 * 7 tokens per step with MTP heads). The T tokens must already be in the cache (appended as usual); query t
 * (0 <= t < T) of sequence i sits at position len - T + t and attends causally to positions
 * [0, len - T + t]: out[i][t][h][:] as kvq_decode_attn over that prefix (body rows before body_len, ring rows
 * after). q_bf16: device bf16 [n_seqs][T][Hq][D]; out: device fp32 [n_seqs][T][Hq][D]; workspace:
 * kvq_workspace_bytes(cache, n_seqs * T, max len) bytes. The cache is not changed; rejected drafts are
 * dropped afterwards with kvq_seq_truncate, which requires them to still be ring rows: tail_len >= T - 1, and
 * any kvq_tail_evict (or fused step) comes after the verification, not before it. With KVQ_LAYOUT_TILES
 * and T >= 2 one multi-query launch reads and decodes every tile of a sequence once for all T queries (a
 * work-group of 8 waves over a range of the tiles, the decoded operands shared through LDS; two queries per wave,
 * or one with KVarN, a qN_1 body or token-axis K); T = 1 runs exactly as kvq_decode_attn; with KVQ_LAYOUT_ROWS
 * each (sequence, query) pair is an entry of the gather launch.
 * Errors: KVQ_E_INVALID if T is outside [1, KVQ_MAX_QUERIES] or n_seqs * T > KVQ_MAX_BATCH; KVQ_E_STATE if
 * a sequence holds fewer than T positions; others as kvq_decode_attn. */
kvq_status kvq_decode_attn_multi(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                 int32_t n_queries, const void* q_bf16, float* out, float softmax_scale,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Chunked prefill: append n_new[i] tokens to each listed sequence (exactly as kvq_append, which quantizes them
 * into the ring and body) and compute causal attention for their queries over the cache as it then stands: the
 * query of new token j of sequence i sits at position p = len_i + j (len_i: the length before the call) and
 * attends to positions [0, p] through the stored representation of every position, the chunk's own tokens
 * included (the KVarN benchmark page and the Qwen3.8-27B page measure prompt processing per cache type).
 * k_bf16, v_bf16: device bf16 [sum n_new][Hkv][D]; q_bf16: device bf16 [sum n_new][Hq][D]; out: device fp32
 * [sum n_new][Hq][D]; all packed in call order. Queries run in blocks of 16 (8 with KVarN, a qN_1 body or
 * token-axis K) through the multi-query kernel, each tile read and decoded once per block. workspace: kvq_prefill_workspace_bytes(cache, n_seqs, max n_new, max
 * length after the call) bytes, 256-byte aligned (NULL allowed when that size is 256).
 * Errors: as kvq_append; KVQ_E_INVALID for a KVQ_LAYOUT_ROWS cache; KVQ_E_SIZE if the workspace is too small
 * (checked before anything is appended). */
kvq_status kvq_prefill_attn(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const int32_t* n_new, const void* k_bf16, const void* v_bf16, const void* q_bf16,
                            float* out, float softmax_scale, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes kvq_prefill_attn needs for n_seqs sequences of at most max_new new tokens and max_len positions
 * after the call (at least 256; 0 for invalid arguments). */
size_t kvq_prefill_workspace_bytes(const kvq_cache* cache, int32_t n_seqs, int32_t max_new, int32_t max_len);

/* Sparse decode attention over an indexer budget (offload page, QSA: the layer reads only the
 * main-KV rows at the positions the indexer chose, so the budget, not the context, bounds the bytes).
 * positions: device int32 [n_seqs][budget], one list per sequence shared by all KV heads; entries are
 * expected to be distinct and in [0, len): entries outside [0, len) are skipped, a repeated entry counts
 * as often as it appears. If no entry of a sequence is valid its output is zero. 1 <= budget.
 * The cache must use KVQ_LAYOUT_ROWS (KVQ_E_INVALID otherwise). Other arguments as kvq_decode_attn;
 * the workspace must hold kvq_workspace_bytes(cache, n_seqs, budget) bytes. */
kvq_status kvq_sparse_decode_attn(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                  const void* q_bf16, const int32_t* positions, int32_t budget, float* out,
                                  float softmax_scale, void* workspace, size_t ws_bytes, void* stream);

/* One sparse decode step of every listed sequence: append one token each (k_bf16, v_bf16: device bf16
 * [n_seqs][Hkv][D]), then sparse decode attention over positions (which index the cache after the append:
 * the new token is at the old length), with the results of kvq_append (n_new = 1 each) followed by
 * kvq_sparse_decode_attn. Without a tail ring and with no KVarN calibration pending, the new rows are
 * quantized into the body inside the sparse decode launch (every work-group whose list range holds the new
 * position builds its rows in LDS and reads that entry from there; the first work-group of each KV head writes
 * them to the body after its own work, and no work-group of the launch reads them from the body); otherwise the
 * calls run in turn. Arguments and errors as those calls; the workspace size
 * (kvq_workspace_bytes(cache, n_seqs, budget)) is checked before any write. */
kvq_status kvq_sparse_decode_step(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                                  const void* k_bf16, const void* v_bf16, const void* q_bf16,
                                  const int32_t* positions, int32_t budget, float* out, float softmax_scale,
                                  void* workspace, size_t ws_bytes, void* stream);

/* ---- The QSA indexer (offload page, QSA paragraph: a cheap indexer runs over keys pooled to
 * indexer_head_dim / indexer_compress_ratio = 128 / 4 = 32 values, picks at most indexer_budget = 2,048
 * positions, and the layer reads only the main-KV rows there; what stays resident is the pooled key, 1 x (128/4)
 * x 2 = 64 bytes per token and layer). A cache with index_dim > 0 holds one pooled key per position. */

/* Pool and store the indexer keys of the newest n_new[i] positions of each listed sequence (call it after the
 * kvq_append that added them). key_bf16: device bf16 [sum n_new][index_dim], sequences packed in call order.
 * Each group of index_pool consecutive values becomes their mean (fp32 sum in order, times 1 / index_pool),
 * rounded to bf16 (nearest even).
 * Errors: KVQ_E_INVALID if the cache has no indexer (index_dim == 0); KVQ_E_STATE if n_new[i] exceeds the
 * sequence's length. */
kvq_status kvq_index_write(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                           const int32_t* n_new, const void* key_bf16, void* stream);

/* Workspace bytes kvq_index_select needs for n_seqs sequences of at most max_len positions. */
size_t kvq_index_workspace_bytes(const kvq_cache* cache, int32_t n_seqs, int32_t max_len);

/* Choose `budget` positions per sequence for sparse decode: the newest n_recent positions, then, of the older
 * positions, those whose pooled key scores highest against the sequence's index query (equal scores: the lower
 * position first). The score of position t is the sum over i = 0..31 of q_i * k_ti, each product exact in fp32
 * and the sum taken in fp32 in channel order, so the choice is reproducible bit for bit. A sequence with no more
 * than `budget` positions has all of them chosen.
 * query_bf16: device bf16 [n_seqs][32]. positions: device int32 [n_seqs][budget], written in ascending order,
 * padded with -1 (entries kvq_sparse_decode_attn skips) when a sequence holds fewer than budget positions.
 * workspace: device, kvq_index_workspace_bytes(cache, n_seqs, max len) bytes, 256-byte aligned, no initial
 * contents needed. Five kernel launches.
 * Errors: KVQ_E_INVALID if the cache has no indexer, budget < 1 or n_recent is outside [0, budget];
 * KVQ_E_SIZE if the workspace is too small. */
kvq_status kvq_index_select(kvq_cache* cache, int32_t layer, int32_t n_seqs, const int32_t* seq_ids,
                            const void* query_bf16, int32_t budget, int32_t n_recent, int32_t* positions,
                            void* workspace, size_t ws_bytes, void* stream);

/* Kernel kinds for launch timing. */
typedef enum {
  KVQ_KERNEL_DECODE = 0,   /* split kernel of dense decode (tile layout)                      */
  KVQ_KERNEL_GATHER = 1,   /* gather kernel of sparse decode / dense decode of a row layout     */
  KVQ_KERNEL_COMBINE = 2,  /* merge of the split partials                                      */
  KVQ_KERNEL_APPEND = 3,   /* append kernels (calibration, body and ring writes, index key writes) */
  KVQ_KERNEL_EVICT = 4,    /* tail-evict requantization                                         */
  KVQ_KERNEL_APPEND_EVICT = 5, /* fused append + evict of kvq_append_evict                        */
  KVQ_KERNEL_INDEX = 6,    /* kvq_index_select, from the start of its scoring launch to the end of its
                              picking launch                                                          */
  KVQ_KERNEL_MQ = 7,       /* multi-query kernel (kvq_decode_attn_multi with T >= 2, kvq_prefill_attn) */
  KVQ_KERNEL_COUNT = 8
} kvq_kernel;

/* Launch timing, for measuring kernels against the memory roofline. While enabled, every launch the
 * handle makes carries a pair of HIP events that the dispatch itself stamps with the kernel's start and
 * end time (hipExtLaunchKernel; host-side objects, no device memory). Enabling or disabling drops earlier
 * records. At most 65,536 launches per kind are recorded; later ones run untimed. */
kvq_status kvq_timing_enable(kvq_cache* cache, int32_t enable);

/* Sum of the recorded launch durations of one kernel kind, in ms, and the number of launches. Waits for
 * the recorded events to complete. */
kvq_status kvq_timing_read(kvq_cache* cache, int32_t kernel, double* total_ms, int32_t* launches);

/* Thread-local text of the last error (never NULL). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
