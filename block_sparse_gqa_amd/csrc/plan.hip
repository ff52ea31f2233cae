// Block -> query inverted index and combine map for the KV-outer schedule.
//
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell" (section 2): the attention kernel
// writes partial outputs contiguously in work order and an index (query, kv head, slot) ->
// location lets the combine kernel gather them; a deterministic, atomic-free scheduler
// flattens all (kv head, kv block, query) work into one sequence. "Sparse Attention"
// (Chapter 5, reverse index): for each block, the queries that chose it, and each one's
// place in the query's list.
//
// Entries are the valid (query, group, block) triples, ordered by (sequence, group, block,
// query). The order is fixed by bitmaps rather than by atomics:
//  1. plan_mask: bucket (s, g, b) gets one 64-bit word per 64 queries, bit i set when query
//     64w + i listed block b (LDS atomics only set bits, so the result is order-free);
//  2. a three-pass exclusive scan of the word popcounts gives every word's first entry;
//  3. plan_scatter: an entry's index is its word's offset plus the popcount of the lower
//     bits; it records the query row and fills the combine map;
//  4. (bf16 attention) plan_tiles / plan_records: each bucket's entries are cut into tiles of
//     256 / group entries (one tile = 256 Q rows of one block), numbered per (s, group, range)
//     phase, and every tile gets a record (first entry, block, entry count) in phase order.
#include <algorithm>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct PlanArgs {
  const int32_t* lists;
  const int32_t* cu_q;
  const int32_t* cu_k;
  unsigned long long* masks;
  const int32_t* offsets;
  int32_t* entry_q;
  int32_t* entry_bucket;
  int32_t* cmap;
  int total_q, total_k, max_q, max_k;
  int hkv, topk, list_q, tiles_max, nb_max, w_max, wr, n_r, wpb, causal;
};

// Bucket (s, h, r, b) of query word w (r = w / wr) and the word's index in the mask array.
__device__ __forceinline__ size_t bucket_of(const PlanArgs& a, int s, int h, int w, int b) {
  return (((size_t)s * a.hkv + h) * a.n_r + w / a.wr) * a.nb_max + b;
}
__device__ __forceinline__ size_t word_index(const PlanArgs& a, int s, int h, int w, int b) {
  return bucket_of(a, s, h, w, b) * a.wr + (w % a.wr);
}

__device__ __forceinline__ const int32_t* list_of(const PlanArgs& a, int s, const Seq& sq,
                                                  int il, int h) {
  const int64_t row = a.list_q == 1 ? (int64_t)(sq.q0 + il)
                                    : (int64_t)s * a.tiles_max + il / a.list_q;
  return a.lists + (row * a.hkv + h) * a.topk;
}

// The entry blocks of one (query, group) list: blk[k] = the block of slot k when it is a real
// entry (in range, first occurrence in the list, and, causally, holding at least one key at or
// before the query's position), else -1. One read of the list row per query.
__device__ __forceinline__ void entry_blocks(const PlanArgs& a, const Seq& sq, int s, int il,
                                             int h, int blk[kMaxTopK]) {
  const int32_t* L = list_of(a, s, sq, il, h);
  const int nb = min((sq.nk + kBlock - 1) / kBlock, a.nb_max);
  const int pos = sq.nk - sq.nq + il;
  int raw[kMaxTopK];
  if (a.topk == kMaxTopK && ((uintptr_t)L & 15) == 0) {
    // a whole 64-byte list row in four 16-byte loads
#pragma unroll
    for (int c = 0; c < kMaxTopK / 4; ++c) {
      const int4 v = reinterpret_cast<const int4*>(L)[c];
      raw[4 * c] = v.x;
      raw[4 * c + 1] = v.y;
      raw[4 * c + 2] = v.z;
      raw[4 * c + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) raw[k] = k < a.topk ? L[k] : -1;
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    const int b = raw[k];
    bool ok = b >= 0 && b < nb && !(a.causal && b * kBlock > pos);
#pragma unroll
    for (int p = 0; p < k; ++p) ok = ok && raw[p] != b;
    blk[k] = ok ? b : -1;
  }
}

// One thread per query of the workgroup's wpb words.
__global__ __launch_bounds__(256) void plan_mask_kernel(PlanArgs a) {
  extern __shared__ unsigned long long lm[];   // [nb_max][wpb]
  const int s = blockIdx.z, h = blockIdx.y;
  const int w0 = blockIdx.x * a.wpb;
  const int tid = threadIdx.x;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int n_lm = a.nb_max * a.wpb;
  for (int i = tid; i < n_lm; i += 256) lm[i] = 0ull;
  __syncthreads();
  const int qa = w0 * kWordQ;
  const int qb = min((w0 + a.wpb) * kWordQ, sq.nq);
  for (int il = qa + tid; il < qb; il += 256) {
    int blk[kMaxTopK];
    entry_blocks(a, sq, s, il, h, blk);
    const unsigned long long bit = 1ull << (il % kWordQ);
    const int wl = il / kWordQ - w0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
      if (blk[k] >= 0) atomicOr(&lm[blk[k] * a.wpb + wl], bit);
  }
  __syncthreads();
  // a workgroup's words lie in one range (wpb divides wr), so each block's words are contiguous
  for (int i = tid; i < n_lm; i += 256) {
    const int b = i / a.wpb, wl = i % a.wpb;
    const int w = w0 + wl;
    if (w < a.n_r * a.wr) a.masks[word_index(a, s, h, w, b)] = lm[i];
  }
}

__global__ __launch_bounds__(256) void plan_scatter_kernel(PlanArgs a) {
  const int s = blockIdx.z, h = blockIdx.y;
  const int w0 = blockIdx.x * a.wpb;
  const int tid = threadIdx.x;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int qa = w0 * kWordQ;
  const int qb = min((w0 + a.wpb) * kWordQ, sq.nq);
  for (int il = qa + tid; il < qb; il += 256) {
    int blk[kMaxTopK];
    entry_blocks(a, sq, s, il, h, blk);
    const int w = il / kWordQ;
    const unsigned long long below = (1ull << (il % kWordQ)) - 1ull;
    int32_t* cm = a.cmap + ((size_t)(sq.q0 + il) * a.hkv + h) * a.topk;
    int ent[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      int e = -1;
      if (blk[k] >= 0) {
        const size_t wi = word_index(a, s, h, w, blk[k]);
        e = a.offsets[wi] + __popcll(a.masks[wi] & below);
        a.entry_q[e] = sq.q0 + il;
        a.entry_bucket[e] = (int)bucket_of(a, s, h, w, blk[k]);
      }
      ent[k] = e;
    }
    if (a.topk == kMaxTopK && ((uintptr_t)cm & 15) == 0) {
#pragma unroll
      for (int c = 0; c < kMaxTopK / 4; ++c)
        reinterpret_cast<int4*>(cm)[c] = make_int4(ent[4 * c], ent[4 * c + 1], ent[4 * c + 2],
                                                   ent[4 * c + 3]);
    } else {
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k)
        if (k < a.topk) cm[k] = ent[k];
    }
  }
}

// ---- three-pass exclusive scan of popcounts (kScanTile words per workgroup)
constexpr int kPer = kScanTile / 256;

__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    pre += (w < wave) ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return pre + x - v;
}

// Word popcounts of a tile, summed. Loads are coalesced: word base + 256 i + thread.
__global__ __launch_bounds__(256) void scan_reduce_kernel(const unsigned long long* __restrict__ masks,
                                                          int64_t n_words, int32_t* __restrict__ sums) {
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x;
  int v = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (base + 256 * i < n_words) v += __popcll(masks[base + 256 * i]);
  int tot;
  block_exclusive_scan(v, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}
__global__ __launch_bounds__(256) void scan_top_kernel(int32_t* __restrict__ sums, int64_t n_blocks,
                                                       int32_t* __restrict__ counters,
                                                       int32_t* __restrict__ offsets_end) {
  int carry = 0;
  for (int64_t b0 = 0; b0 < n_blocks; b0 += 256) {
    const int64_t i = b0 + threadIdx.x;
    const int v = i < n_blocks ? sums[i] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, &tot);
    if (i < n_blocks) sums[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    counters[0] = carry;
    *offsets_end = carry;
  }
}

// Offsets of a tile's words: wave w scans words w kScanTile / 4 .. +kScanTile / 4 - 1 of the
// tile in kPer rounds of 64 consecutive words (coalesced loads and stores), carrying the
// running sum from round to round; the waves' totals order the four segments.
__global__ __launch_bounds__(256) void scan_down_kernel(const unsigned long long* __restrict__ masks,
                                                        int64_t n_words, const int32_t* __restrict__ sums,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * kScanTile + wave * (kScanTile / 4) + lane;
  int cnt[kPer];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cnt[i] = (base + 64 * i < n_words) ? __popcll(masks[base + 64 * i]) : 0;
    tot += cnt[i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
  if (lane == 0) wsum[wave] = tot;
  __syncthreads();
  int run = sums[blockIdx.x];
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int x = cnt[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (base + 64 * i < n_words) offsets[base + 64 * i] = run + x - cnt[i];
    run += __shfl(x, 63, 64);
  }
}


// ---- tiles of the bf16 attention kernel (one workgroup per phase)
struct TileArgs {
  const int32_t* offsets;     // entry offset of every bitmap word (+ E at the end)
  int32_t* tile_off;          // [n_buckets] first tile of each bucket, phase-relative
  int32_t* phase_base;        // [n_phase + 1] first record of each phase
  int32_t* phase_n;           // [n_phase] tiles of each phase
  int2* recs;                 // tile records
  int wr, nb_max, mq, n_phase;
};

__device__ __forceinline__ int bucket_entries(const TileArgs& a, int64_t bk, int* e0) {
  const int b0 = a.offsets[bk * a.wr];
  *e0 = b0;
  return a.offsets[(bk + 1) * a.wr] - b0;
}

// Exclusive scan of the tile counts of the phase's buckets.
__global__ __launch_bounds__(256) void plan_tiles_kernel(TileArgs a) {
  const int p = blockIdx.x, tid = threadIdx.x;
  const int per = (a.nb_max + 255) / 256;          // consecutive buckets per thread (<= 32)
  const int b0 = tid * per;
  int v = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.nb_max) {
      int e0;
      const int c = bucket_entries(a, (int64_t)p * a.nb_max + b, &e0);
      v += (c + a.mq - 1) / a.mq;
    }
  }
  int tot;
  int run = block_exclusive_scan(v, &tot);
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.nb_max) {
      const int64_t bk = (int64_t)p * a.nb_max + b;
      int e0;
      const int c = bucket_entries(a, bk, &e0);
      a.tile_off[bk] = run;
      run += (c + a.mq - 1) / a.mq;
    }
  }
  if (tid == 0) a.phase_n[p] = tot;
}

// Phase bases (sum of the tile counts of the earlier phases) and the tile records.
__global__ __launch_bounds__(256) void plan_records_kernel(TileArgs a) {
  const int p = blockIdx.x, tid = threadIdx.x;
  int v = 0;
  for (int i = tid; i < p; i += 256) v += a.phase_n[i];
  int base;
  block_exclusive_scan(v, &base);                  // base = total over the threads
  if (tid == 0) {
    a.phase_base[p] = base;
    if (p == a.n_phase - 1) a.phase_base[a.n_phase] = base + a.phase_n[p];
  }
  for (int b = tid; b < a.nb_max; b += 256) {
    const int64_t bk = (int64_t)p * a.nb_max + b;
    int e0;
    const int c = bucket_entries(a, bk, &e0);
    const int t0 = base + a.tile_off[bk];
    for (int i = 0; i * a.mq < c; ++i) {
      const int n = min(a.mq, c - i * a.mq);
      a.recs[t0 + i] = make_int2(e0 + i * a.mq, (b << 8) | (n - 1));
    }
  }
}
}  // namespace

hipError_t launch_plan(const msa_shape& s, const Geometry& g, const Layout& L,
                       const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k,
                       char* ws, hipStream_t st) {
  PlanArgs a;
  a.lists = lists;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.masks = reinterpret_cast<unsigned long long*>(ws + L.masks);
  a.offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  a.entry_q = reinterpret_cast<int32_t*>(ws + L.entry_q);
  a.entry_bucket = reinterpret_cast<int32_t*>(ws + L.entry_bucket);
  a.cmap = reinterpret_cast<int32_t*>(ws + L.cmap);
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.hkv = s.hkv;
  a.topk = s.topk;
  a.list_q = s.list_q;
  a.tiles_max = (int)g.tiles_max;
  a.nb_max = (int)g.nb_max;
  a.w_max = (int)g.w_max;
  a.wr = (int)g.wr;
  a.n_r = (int)g.n_r;
  a.causal = s.causal;
  int32_t* counters = reinterpret_cast<int32_t*>(ws + L.counters);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sums = reinterpret_cast<int32_t*>(ws + L.scan_sums);

  if (g.n_words == 0) {
    // nothing can be selected: zero entries
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, st, sums, (int64_t)0, counters,
                       offsets);
    return hipGetLastError();
  }
  // words per workgroup: keep the LDS bitmap tile at <= 64 KiB
  // (powers of two, so that wpb divides wr and a workgroup stays inside one range)
  int wpb = 8;
  while (wpb > 1 && (int64_t)wpb * g.nb_max > 8192) wpb >>= 1;
  while (wpb > g.wr) wpb >>= 1;
  a.wpb = wpb;
  const size_t lds = (size_t)g.nb_max * wpb * 8;
  dim3 grid((unsigned)((g.n_r * g.wr) / wpb), s.hkv, s.batch);
  hipLaunchKernelGGL(plan_mask_kernel, grid, dim3(256), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nblk = (unsigned)g.n_scan_blocks;
  hipLaunchKernelGGL(scan_reduce_kernel, dim3(nblk), dim3(256), 0, st,
                     (const unsigned long long*)a.masks, (int64_t)g.n_words, sums);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, st, sums, (int64_t)nblk, counters,
                     offsets + g.n_words);
  hipLaunchKernelGGL(scan_down_kernel, dim3(nblk), dim3(256), 0, st,
                     (const unsigned long long*)a.masks, (int64_t)g.n_words,
                     (const int32_t*)sums, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_scatter_kernel, grid, dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TileArgs t;
  t.offsets = offsets;
  t.tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
  t.phase_base = reinterpret_cast<int32_t*>(ws + L.phase_base);
  t.phase_n = t.phase_base + g.n_phase + 1;
  t.recs = reinterpret_cast<int2*>(ws + L.tiles);
  t.wr = (int)g.wr;
  t.nb_max = (int)g.nb_max;
  t.mq = 256 / g.group;
  t.n_phase = (int)g.n_phase;
  hipLaunchKernelGGL(plan_tiles_kernel, dim3((unsigned)g.n_phase), dim3(256), 0, st, t);
  hipLaunchKernelGGL(plan_records_kernel, dim3((unsigned)g.n_phase), dim3(256), 0, st, t);
  return hipGetLastError();
}

}  // namespace msa
