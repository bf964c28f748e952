// The QSA indexer: pooled index keys, their scores against an index query, and the choice of a budget of
// positions for sparse decode (offload page, QSA paragraph: a cheap indexer runs over keys pooled to
// indexer_head_dim / indexer_compress_ratio = 128 / 4 = 32 values; it picks at most indexer_budget positions
// and the layer reads only the main-KV rows there; what stays resident is 1 x (128 / 4) x 2 = 64 bytes of
// pooled key per token and layer).
//
// Scoring is a 32-term dot product per position over 64 bytes of key: HBM-bound, so it runs on the VALU (one
// position per thread), not on matrix cores. The score is defined bit for bit (products exact in fp32, summed
// in channel order) so that the chosen set is reproducible; contraction is off in this file.
//
// Selection of the top k of m scores in five launches; each hands its results to the next through the kernel
// boundary (on this GPU a device-scope fence inside a kernel writes back the XCD's L2, so work-groups do not hand
// data to one another within a launch):
//   zero_kernel       clears the per-sequence histograms and counters in the workspace;
//   score_kernel      four positions per thread: the score, its order-preserving 32-bit key (stored), and a
//                     16,384-bin histogram of the key's top 14 bits (in LDS, then added to one of the sequence's
//                     histogram copies);
//   threshold_kernel  one work-group per sequence: the bin that holds the k-th largest key;
//   classify_kernel   four positions per thread: positions above that bin are chosen (a bitmap written by wave
//                     ballots), positions in it become candidates;
//   finalize_kernel   one work-group per sequence: the needed number of candidates by an exact radix select on
//                     (key, lower position first), then the bitmap compacted into the ascending position list,
//                     then the newest n_recent positions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_kernels.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kIdxThreads = 1024;                       // threads of the score and pick kernels
constexpr int kIdxPerThread = kIndexChunk / kIdxThreads;   // positions per thread
constexpr int kHistBits = 14;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kLowBits = 32 - kHistBits;  // key bits below the histogram bin

// Per-sequence control words in the workspace (after the histogram).
enum { kCtlBin = 0, kCtlNeed, kCtlCand, kCtlWords = 16 };
// Threshold bin values beyond any histogram bin: every scored position chosen, or none.
constexpr uint32_t kBinAll = 0xFFFFFFFFu, kBinNone = 0xFFFFFFFEu;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Order-preserving key of a finite fp32 score (+0 and -0 are the same score: -0 is made +0 first).
__device__ inline uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The work-group's sequence and chunk (work-groups are laid out sequence after sequence).
__device__ inline int seq_of(const IndexArgs& a, int wg) {
  int s = 0;
  while (s + 1 < a.n_seqs && a.seqs[s + 1].wg_begin <= wg) ++s;
  return s;
}

__device__ inline uint32_t* hist_of(const IndexArgs& a, int s) { return (uint32_t*)(a.ws + a.seqs[s].ws_off); }
__device__ inline uint32_t* ctl_of(const IndexArgs& a, int s) { return hist_of(a, s) + kIndexHistCopies * kHistBins; }
__device__ inline uint32_t* keys_of(const IndexArgs& a, int s) { return ctl_of(a, s) + kCtlWords; }
__device__ inline uint32_t* bitmap_of(const IndexArgs& a, int s) {
  return keys_of(a, s) + (size_t)a.seqs[s].n_wgs * kIndexChunk;
}
__device__ inline uint2* cand_of(const IndexArgs& a, int s) {
  return (uint2*)(bitmap_of(a, s) + (size_t)a.seqs[s].n_wgs * (kIndexChunk / 32));
}

// Block-wide exclusive prefix sum of one value per thread (1024 threads); *total receives the sum. Wave sums by
// shuffles, then the 16 wave totals scanned by shuffles within wave 0.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kIdxThreads / 64;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t t = lane < kWaves ? s_tmp[lane] : 0u;
    uint32_t u = t;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const uint32_t y = __shfl_up(u, o);
      if (lane >= o) u += y;
    }
    if (lane < kWaves) s_tmp[lane] = u - t;          // exclusive prefix of the wave totals
    if (lane == kWaves - 1) s_tmp[kWaves] = u;        // the block total
  }
  __syncthreads();
  const uint32_t r = x - v + s_tmp[wave];
  *total = s_tmp[kWaves];
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------------------------------- index write

// One work-group of 256 threads per 8 positions: thread (position, i) pools values i*pool .. i*pool + pool - 1
// of the position's indexer key (fp32 sum in order, times 1/pool, round to nearest even bf16).
__global__ __launch_bounds__(256) void index_write_kernel(IndexWriteArgs a) {
  const int tid = threadIdx.x;
  const int q = blockIdx.x * 8 + (tid >> 5);   // position number over all items
  const int i = tid & 31;
  int it = 0;
  while (it + 1 < a.n_items && a.items[it + 1].begin <= q) ++it;
  const IndexWriteItem& w = a.items[it];
  if (q >= w.begin + w.n) return;
  const int k = q - w.begin;
  const uint16_t* src = a.key_in + (size_t)(w.row0 + k) * (kIndexWidth * a.pool) + i * a.pool;
  float s = bf16f(src[0]);
  for (int j = 1; j < a.pool; ++j) s = s + bf16f(src[j]);
  const float mean = s * (1.0f / (float)a.pool);    // exact: pool is a power of two
  const uint32_t u = __float_as_uint(mean);
  const uint16_t b = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  uint16_t* dst = (uint16_t*)(a.g.arena + w.slab + a.g.index) + (size_t)(w.p0 + k) * kIndexWidth;
  dst[i] = b;
}

// ------------------------------------------------------------------------------------------- selection

// Position r of thread tid in a work-group's chunk (4 positions per thread, each row of 1,024 coalesced).
__device__ inline int chunk_pos(int wg_in_seq, int r, int tid) { return wg_in_seq * kIndexChunk + r * kIdxThreads + tid; }

// Global histogram: kHistCopies copies (work-group w adds into copy w % kHistCopies), each with its bins
// interleaved so that neighbouring bins (scores of similar size, added by every work-group) sit on different
// cache lines: fewer atomics meet on one line.
constexpr int kHistCopies = kIndexHistCopies;
__device__ inline int hist_slot(int bin) { return ((bin & 127) << 7) | (bin >> 7); }

__global__ __launch_bounds__(1024) void index_zero_kernel(IndexArgs a) {
  uint32_t* h = hist_of(a, blockIdx.x);
  for (int i = threadIdx.x; i < kHistCopies * kHistBins + kCtlWords; i += blockDim.x) h[i] = 0u;
}

__global__ __launch_bounds__(1024) void index_score_kernel(IndexArgs a) {
  __shared__ uint32_t s_hist[kHistBins];
  const int wg = blockIdx.x;
  const int si = seq_of(a, wg);
  const IndexSeq& S = a.seqs[si];
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += kIdxThreads) s_hist[i] = 0u;
  // the query: 32 bf16 values (a uniform address)
  const uint16_t* qp = a.q + (size_t)si * kIndexWidth;
  float q[kIndexWidth];
#pragma unroll
  for (int i = 0; i < kIndexWidth; ++i) q[i] = bf16f(qp[i]);
  __syncthreads();
  uint32_t* keys = keys_of(a, si);
#pragma unroll
  for (int r = 0; r < kIdxPerThread; ++r) {
    const int t = chunk_pos(wg - S.wg_begin, r, tid);
    if (t < S.m) {
      const u32x4* kp = (const u32x4*)(a.g.arena + S.slab + a.g.index + (size_t)t * (2 * kIndexWidth));
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = kp[j];   // cached: the four loads of a wave share their lines
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v[4] = {w[j][0], w[j][1], w[j][2], w[j][3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = acc + q[8 * j + 2 * e] * __uint_as_float(v[e] << 16);               // exact product, then round
          acc = acc + q[8 * j + 2 * e + 1] * __uint_as_float(v[e] & 0xFFFF0000u);
        }
      }
      const uint32_t key = score_key(acc);
      keys[t] = key;
      atomicAdd(&s_hist[key >> kLowBits], 1u);
    }
  }
  __syncthreads();
  uint32_t* gc = hist_of(a, si) + ((wg - S.wg_begin) % kHistCopies) * kHistBins;
  for (int i = tid; i < kHistBins; i += kIdxThreads)
    if (s_hist[i]) atomicAdd(&gc[hist_slot(i)], s_hist[i]);
}

// One work-group per sequence: the bin that holds the k-th largest key (counted from the top bin down) and how many
// keys are needed from it.
__global__ __launch_bounds__(1024) void index_threshold_kernel(IndexArgs a) {
  __shared__ uint32_t s_cnt[kHistBins + kHistBins / 128];   // bin b at b + b / 128: the transposed stores of a
  __shared__ uint32_t s_tmp[kIdxThreads / 64 + 1];            // wave fall on 64 different banks
  const int si = blockIdx.x;
  const IndexSeq& S = a.seqs[si];
  const int tid = threadIdx.x;
  uint32_t* ctl = ctl_of(a, si);
  if (S.m <= S.k || S.k == 0) {   // every scored position is chosen, or none (the budget is all recent)
    if (tid == 0) {
      ctl[kCtlBin] = S.k == 0 ? kBinNone : kBinAll;
      ctl[kCtlNeed] = 0u;
    }
    return;
  }
  // the copies summed slot by slot (16-byte loads, all issued before any is used), stored in bin order
  const u32x4* gh = (const u32x4*)hist_of(a, si);
  constexpr int kPer = kHistBins / 4 / kIdxThreads;
  u32x4 c[kPer][kHistCopies];
#pragma unroll
  for (int r = 0; r < kPer; ++r)
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) c[r][cp] = gh[cp * (kHistBins / 4) + r * kIdxThreads + tid];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    u32x4 t = c[r][0];
#pragma unroll
    for (int cp = 1; cp < kHistCopies; ++cp) t += c[r][cp];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int slot = 4 * (r * kIdxThreads + tid) + e;
      const int b = ((slot & 127) << 7) | (slot >> 7);   // the slot map is its own inverse
      s_cnt[b + (b >> 7)] = t[e];
    }
  }
  __syncthreads();
  // thread tid covers bins [kHistBins - 16 (tid + 1), kHistBins - 16 tid), the top bins first
  const int hi = kHistBins - 16 * tid;
  uint32_t cnt[16];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int b = hi - 1 - j;
    cnt[j] = s_cnt[b + (b >> 7)];
    sum += cnt[j];
  }
  uint32_t total;
  const uint32_t above = block_exclusive_scan(sum, s_tmp, &total);   // keys in bins above this thread's
  const uint32_t k = (uint32_t)S.k;
  if (above < k && above + sum >= k) {
    uint32_t acc = above;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (acc + cnt[j] >= k) {
        ctl[kCtlBin] = (uint32_t)(hi - 1 - j);
        ctl[kCtlNeed] = k - acc;   // keys needed from this bin
        break;
      }
      acc += cnt[j];
    }
  }
}

// Positions above the threshold bin are chosen (a bitmap written by wave ballots: each wave owns the two words of
// its 64 positions); positions in the bin become candidates.
__global__ __launch_bounds__(1024) void index_classify_kernel(IndexArgs a) {
  const int wg = blockIdx.x;
  const int si = seq_of(a, wg);
  const IndexSeq& S = a.seqs[si];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  uint32_t* ctl = ctl_of(a, si);
  const uint32_t bin = ctl[kCtlBin];
  const bool all = bin == kBinAll, none = bin == kBinNone;
  uint32_t* bm = bitmap_of(a, si);
  const uint32_t* keys = keys_of(a, si);
#pragma unroll
  for (int r = 0; r < kIdxPerThread; ++r) {
    const int t = chunk_pos(wg - S.wg_begin, r, tid);
    const bool valid = t < S.m;
    uint32_t key = 0;
    if (valid) key = keys[t];
    const uint32_t kb = key >> kLowBits;
    const bool sel = valid && (all || (!none && kb > bin));
    const bool cand = valid && !all && !none && kb == bin;
    const uint64_t bs = __ballot(sel);
    if (lane == 0) {
      bm[t >> 5] = (uint32_t)bs;
      bm[(t >> 5) + 1] = (uint32_t)(bs >> 32);
    }
    const uint64_t bc = __ballot(cand);
    if (bc) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&ctl[kCtlCand], (uint32_t)__popcll(bc));
      base = __shfl(base, 0);
      if (cand) {
        const uint32_t rk = (uint32_t)__popcll(bc & ((1ull << lane) - 1ull));
        cand_of(a, si)[base + rk] = make_uint2(key & ((1u << kLowBits) - 1u), (uint32_t)t);
      }
    }
  }
}

// One work-group per sequence: pick `need` candidates by an exact radix select on the composite (low key bits,
// then the lower position first), i.e. on c = (lowkey << 32) | ~position, largest first; then compact the bitmap
// into the ascending position list, append the newest positions and pad.
constexpr int kCandLds = 8192;   // candidates the finalize work-group keeps in LDS (more: read from global memory)

__global__ __launch_bounds__(1024) void index_finalize_kernel(IndexArgs a) {
  __shared__ uint32_t s_tmp[kIdxThreads / 64 + 1];
  __shared__ uint32_t s_h[256];
  __shared__ uint32_t s_sel[4];
  __shared__ uint2 s_cand[kCandLds];
  const int si = blockIdx.x;
  const IndexSeq& S = a.seqs[si];
  const int tid = threadIdx.x;
  uint32_t* ctl = ctl_of(a, si);
  const uint32_t bin = ctl[kCtlBin];
  uint32_t* bm = bitmap_of(a, si);
  if (bin != kBinAll && bin != kBinNone) {
    uint32_t need = ctl[kCtlNeed];
    const uint32_t nc = ctl[kCtlCand];
    const uint2* cd = cand_of(a, si);
    if (nc <= (uint32_t)kCandLds) {   // the passes below then read LDS, not global memory
      for (uint32_t i = tid; i < nc; i += kIdxThreads) s_cand[i] = cd[i];
      __syncthreads();
      cd = s_cand;
    }
    if (nc <= (uint32_t)kIdxThreads) {
      // few candidates: each thread counts the candidates that outrank its own (larger composite); the `need`
      // candidates outranked by fewer than `need` others are chosen
      if ((uint32_t)tid < nc) {
        const uint2 me = cd[tid];
        const uint64_t cm = ((uint64_t)me.x << 32) | (uint32_t)~me.y;
        uint32_t beat = 0;
        for (uint32_t i = 0; i < nc; ++i) {
          const uint2 e = cd[i];
          beat += (((uint64_t)e.x << 32) | (uint32_t)~e.y) > cm ? 1u : 0u;
        }
        if (beat < need) atomicOr(&bm[me.y >> 5], 1u << (me.y & 31));
      }
      need = 0;   // done: the radix passes below are skipped
    }
    if (need > 0) {
    // digits of the 50-bit composite from the top: bits 49..42, 41..34, ..., 9..2, 1..0
    uint64_t prefix = 0, pmask = 0;
    for (int shift = 42; shift >= -6; shift -= 8) {
      const int sh = shift < 0 ? 0 : shift;
      const int width = shift < 0 ? 8 + shift : 8;
      for (int i = tid; i < 256; i += kIdxThreads) s_h[i] = 0u;
      __syncthreads();
      const uint64_t dmask = ((1ull << width) - 1ull) << sh;
      for (uint32_t i = tid; i < nc; i += kIdxThreads) {
        const uint2 e = cd[i];
        const uint64_t c = ((uint64_t)e.x << 32) | (uint32_t)~e.y;
        if ((c & pmask) == prefix) atomicAdd(&s_h[(c & dmask) >> sh], 1u);
      }
      __syncthreads();
      // the digit holding the need-th largest: thread t takes digit 255 - t, a scan counts from the top digit
      const uint32_t h = tid < 256 ? s_h[255 - tid] : 0u;
      uint32_t tot;
      const uint32_t above = block_exclusive_scan(h, s_tmp, &tot);
      if (tid < 256 && above < need && above + h >= need) {
        s_sel[0] = (uint32_t)(255 - tid);
        s_sel[1] = need - above;
      }
      __syncthreads();
      prefix |= (uint64_t)s_sel[0] << sh;
      pmask |= dmask;
      need = s_sel[1];
      __syncthreads();
    }
    // prefix is now the composite of the last candidate taken: every candidate at or above it is chosen
    for (uint32_t i = tid; i < nc; i += kIdxThreads) {
      const uint2 e = cd[i];
      const uint64_t c = ((uint64_t)e.x << 32) | (uint32_t)~e.y;
      if (c >= prefix) atomicOr(&bm[e.y >> 5], 1u << (e.y & 31));
    }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the bits are set before any wave of this work-group reads the words
    __syncthreads();
  }
  // compaction: the bitmap words in order, 8 consecutive words per thread and pass (two 16-byte loads; words at
  // or past the scored range are zero, and the bitmap is allocated in whole work-groups of 32 words)
  const int n_words = (S.m + 31) / 32;
  int32_t* out = a.out + (size_t)si * a.budget;
  uint32_t n_sel_all = 0;
  for (int wb = 0; wb < n_words; wb += 8 * kIdxThreads) {
    const int w0 = wb + 8 * tid;
    u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
    if (w0 < n_words) {
      x0 = ((const u32x4*)bm)[w0 / 4];
      x1 = ((const u32x4*)bm)[w0 / 4 + 1];
    }
    const uint32_t x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) cnt += (uint32_t)__popc(x[j]);
    uint32_t total;
    uint32_t off = n_sel_all + block_exclusive_scan(cnt, s_tmp, &total);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t y = x[j];
      while (y) {
        const int b = __builtin_ctz(y);
        y &= y - 1;
        if (off < (uint32_t)a.budget) out[off] = 32 * (w0 + j) + b;   // the bitmap holds at most k <= budget bits
        ++off;
      }
    }
    n_sel_all += total;
  }
  // then the newest positions, then padding
  const int n_sel = min((int)n_sel_all, a.budget);
  for (int i = tid; i < a.budget - n_sel; i += kIdxThreads) {
    const int p = S.m + i;
    out[n_sel + i] = p < S.len ? p : -1;
  }
}

}  // namespace

hipError_t launch_index_write(const IndexWriteArgs& a, int n_positions, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  return launch_k(index_write_kernel, dim3((n_positions + 7) / 8), dim3(256), s, e0, e1, a);
}

hipError_t launch_index_select(const IndexArgs& a, int total_wgs, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 blk(kIdxThreads);
  hipError_t e = launch_k(index_zero_kernel, dim3(a.n_seqs), blk, s, nullptr, nullptr, a);
  if (e != hipSuccess) return e;
  // with timing, the scoring launch stamps e0 with its start and the finishing launch e1 with its end
  if (e0) hipExtLaunchKernelGGL(index_score_kernel, dim3(total_wgs), blk, 0, s, e0, nullptr, 0, a);
  else hipLaunchKernelGGL(index_score_kernel, dim3(total_wgs), blk, 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_k(index_threshold_kernel, dim3(a.n_seqs), blk, s, nullptr, nullptr, a)) != hipSuccess) return e;
  if ((e = launch_k(index_classify_kernel, dim3(total_wgs), blk, s, nullptr, nullptr, a)) != hipSuccess) return e;
  if (e1) hipExtLaunchKernelGGL(index_finalize_kernel, dim3(a.n_seqs), blk, 0, s, nullptr, e1, 0, a);
  else hipLaunchKernelGGL(index_finalize_kernel, dim3(a.n_seqs), blk, 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
