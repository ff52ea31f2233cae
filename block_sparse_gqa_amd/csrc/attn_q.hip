// Q-outer (query-stationary) sparse attention: the low-reuse schedule.
//
// "Sparse Attention" (Chapter 2): a query tile walks selected_indices[base + slot] for
// slot < selected_count, running the usual load K/V, QK, online-softmax, PV step per block.
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell" (section 1): this structure
// re-reads blocks through the cache instead of writing partials, and wins when few queries
// share each block (high nsb/N, e.g. decode).
//
// A workgroup owns the rows that share one list: the 128 queries of a Q tile for one head
// (per-tile lists), or the G heads of one query (per-query lists). The rows' Q stays in
// registers; each listed block is staged in LDS and folded in with an online softmax.
// Per-query lists may be split over `splits` workgroups, each writing a partial that the
// combine kernel merges.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct QArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* descale;
  float scale_log2;
  const int32_t* lists;
  const int32_t* cu_q;
  const int32_t* cu_k;
  uint16_t* o;
  float* lse;
  int32_t* counters;
  int32_t* cmap;
  float* part_lse;
  float* part_l;
  uint16_t* part_o;
  int total_q, total_k, max_q, max_k;
  int batch, hq, hkv, topk, list_q, tiles_max, causal, splits;
};

__device__ __forceinline__ int seq_of_row(const int32_t* cu_q, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Per-tile lists: (tile, head) of linear workgroup id `id` over a tiles x heads grid. The
// hardware hands ids to the 8 XCDs round-robin; XCD x = id % 8 takes the (id / 8)-th pair of
// its own contiguous run of head-major (head, tile) pairs, so the workgroups running together
// on one XCD share heads and their K/V blocks stay in that XCD's L2.
__device__ __forceinline__ void xcd_tile_head(int id, int tiles, int heads, int* tile,
                                              int* head) {
  const int n = tiles * heads;
  int pair = id;
  if (n % 8 == 0) pair = (id % 8) * (n / 8) + id / 8;   // a bijection of [0, n)
  *head = pair / tiles;
  *tile = pair % tiles;
}

// The blocks a workgroup visits, in list order: the slots [slot0, slot1) of `list` whose block
// is valid (0 <= b < nb), visible to some row of the workgroup (causal: 128 b <= pos_max) and
// not listed in an earlier slot. Built by one wave, one list entry per lane (topk <= 64).
__device__ __forceinline__ void visit_list(const int32_t* list, int topk, int slot0, int slot1,
                                           int nb, bool causal, int pos_max, int* vis,
                                           int* n_vis) {
  const int lane = threadIdx.x & 63;
  const int b = lane < topk ? list[lane] : -1;
  bool use = lane >= slot0 && lane < slot1 && b >= 0 && b < nb &&
             !(causal && b * kBlock > pos_max);
#pragma unroll
  for (int p = 0; p < kMaxTopK; ++p) {
    const int bp = __shfl(b, p, 64);
    if (p < lane && bp == b) use = false;
  }
  const unsigned long long m = __ballot(use);
  if (use) vis[__popcll(m & ((1ull << lane) - 1))] = b;
  if (lane == 0) *n_vis = __popcll(m);
}

// The same list kept in registers: lane i (< count) of the calling wave receives the i-th
// visited block. Every wave builds its own copy.
__device__ __forceinline__ int visit_list_lanes(const int32_t* list, int topk, int nb,
                                                bool causal, int pos_max, int* count) {
  const int lane = threadIdx.x & 63;
  const int b = lane < topk ? list[lane] : -1;
  bool use = b >= 0 && b < nb && !(causal && b * kBlock > pos_max);
#pragma unroll
  for (int p = 0; p < kMaxTopK; ++p) {
    const int bp = __shfl(b, p, 64);
    if (p < lane && bp == b) use = false;
  }
  const unsigned long long m = __ballot(use);
  *count = __popcll(m);
  // forward permute: a used entry goes to lane (its rank); the others to lanes 32..63
  const int dst = use ? __popcll(m & ((1ull << lane) - 1)) : (32 | (lane & 31));
  return __builtin_amdgcn_ds_permute(dst * 4, b);
}

// fp8 lists (per-tile or per-query): e4m3 K and V are widened to bf16 while staged through
// registers into LDS, one block at a time. bf16 lists run in attn_qd_kernel (per query) and
// attn_qt_kernel (per tile).
template <bool FP8, int G>
__global__ __launch_bounds__(256, 2) void attn_q_kernel(QArgs a) {
  static_assert(FP8, "bf16 lists run in attn_qd_kernel and attn_qt_kernel");
  constexpr int EB = FP8 ? 1 : 2;
  __shared__ KVLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int r = wave * 32 + col;

  // --- the rows of this workgroup and their list
  int s, h, hh, t, split, tile = 0;
  bool valid;
  const int32_t* list;
  if (a.list_q > 1) {
    // Workgroup ids go round-robin over the XCDs; remap them so that the tiles of one head
    // run together on one XCD, whose L2 then holds that head's K/V blocks.
    xcd_tile_head(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x, gridDim.y, &tile, &hh);
    h = hh / G;
    s = blockIdx.z;
    split = 0;
    const Seq sq0 = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
    if (tile * a.list_q >= sq0.nq) return;
    const int il = tile * a.list_q + r;
    valid = r < a.list_q && il < sq0.nq;
    t = sq0.q0 + (valid ? il : 0);
    list = a.lists + (((size_t)s * a.tiles_max + tile) * a.hkv + h) * a.topk;
  } else {
    const int tq = blockIdx.x;
    h = blockIdx.y;
    split = blockIdx.z;
    if (tq >= a.total_q) return;
    s = seq_of_row(a.cu_q, a.batch, tq);
    valid = r < G;
    hh = h * G + (valid ? r : 0);
    t = tq;
    list = a.lists + ((size_t)tq * a.hkv + h) * a.topk;
  }
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  if (t - sq.q0 >= sq.nq) valid = false;      // row past a clamped sequence
  const int pos = sq.nk - sq.nq + (t - sq.q0);
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  // the workgroup's largest position (rows are in query order) for whole-block skipping
  int pos_max;
  if (a.list_q > 1) {
    const int il_last = min(tile * a.list_q + a.list_q - 1, sq.nq - 1);
    pos_max = sq.nk - sq.nq + il_last;
  } else {
    pos_max = pos;
  }
  const bool wave_rows = a.list_q > 1 ? true : (wave * 32 < G);

  float sl2 = a.scale_log2, dv = 1.f;
  if constexpr (FP8) {
    sl2 *= a.descale[0] * a.descale[1];
    dv = a.descale[2];
  }
  const char* qb = reinterpret_cast<const char*>(a.q);
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const uint32_t kv_row = (uint32_t)a.hkv * kD;

  bf16x8 bq[8];
  load_q_operand<FP8>(bq, qb + ((size_t)t * a.hq + hh) * kD * EB, hf);

  const float ninf = -__builtin_inff();
  float m_run = ninf, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  const int per = (a.topk + a.splits - 1) / a.splits;
  const int slot0 = split * per, slot1 = min(a.topk, slot0 + per);
  // The blocks this workgroup visits (uniform): valid, visible to some row, first occurrence.
  __shared__ int vis[kMaxTopK];
  __shared__ int n_vis;
  if (tid < 64) visit_list(list, a.topk, slot0, slot1, nb, a.causal, pos_max, vis, &n_vis);
  __syncthreads();
  const int nv = n_vis;

  auto fold = [&](int u0, int nk_rel, auto&& pv) {
    f32x16 sacc[4];
    qk_block(L, bq, sacc, col, hf);
    int kmax = min(127, nk_rel - 1);
    if (a.causal) kmax = min(kmax, pos - u0);
    const float mb = mask_max(sacc, kmax, __any(kmax < 127), hf);
    const float m_new = fmaxf(m_run, mb);          // raw-score units
    const float c = m_new > ninf ? m_new * sl2 : 0.f;
    const float alpha = m_run > ninf ? __builtin_amdgcn_exp2f(m_run * sl2 - c) : 0.f;
    u32x4 pk[4][2];
    const float lb = exp_pack(sacc, sl2, c, pk);
    l_run = l_run * alpha + lb;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    m_run = m_new;
    pv(pk);
  };

  if constexpr (FP8) {
    // fp8 K/V are widened to bf16 while staging (through registers), one block at a time
    for (int j = 0; j < nv; ++j) {
      const int u0 = vis[j] * kBlock;
      const int nk_rel = sq.nk - u0;
      __syncthreads();
      stage_kv<FP8>(L, kb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB,
                    vb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB, kv_row, nk_rel);
      __syncthreads();
      if (wave_rows) fold(u0, nk_rel, [&](const u32x4 (&pk)[4][2]) {
        pv_block<false>(L, pk, oacc, col, hf);
      });
    }
  }

  if (a.splits > 1 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0)
    a.counters[0] = a.total_q * a.hkv * a.splits;
  if (!valid) return;
  const bool any = l_run > 0.f;
  const float inv = any ? dv / l_run : 0.f;
  const float lse_v = any ? (m_run * sl2 + log2f(l_run)) * 0.69314718055994531f : ninf;
  const int g = hh - h * G;
  if (a.splits == 1) {
    store_o_row(a.o + ((size_t)t * a.hq + hh) * kD, oacc, inv, hf);
    if (hf == 0 && a.lse) a.lse[(size_t)t * a.hq + hh] = lse_v;
  } else {
    const size_t pe = ((size_t)t * a.hkv + h) * a.splits + split;
    store_o_part(a.part_o, pe * G + g, oacc, inv, hf);
    if (hf == 0) {
      a.part_lse[pe * G + g] = lse_v;
      a.part_l[pe * G + g] = 1.f;           // the partial output is already normalised
      if (g == 0) a.cmap[pe] = (int)pe;
    }
  }
}

// Per-query lists, bf16: the G heads of one query over the listed blocks of a split, on two
// waves that take the two key halves of every block (wave w: keys 64 w .. 64 w + 63), each with
// its own running max, sum and output, merged once at the end; K and V are double-buffered in
// LDS (128 KiB, one workgroup per CU). At the top of step j the workgroup waits for block j,
// crosses its one barrier of the step and issues block j + 1 from all four waves, so a whole
// block is in flight while block j is computed. The running max is raised only when a block's
// max exceeds it by more than 2^8 in probability, as in the per-tile kernel below.
template <int G>
__global__ __launch_bounds__(256, 1) void attn_qd_kernel(QArgs a) {
  __shared__ KVLds L[2];
  __shared__ int vis[kMaxTopK];
  __shared__ int n_vis;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const bool math = wave < 2;
  const int kt0 = 2 * (wave & 1);
  const int tq = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
  if (tq >= a.total_q) return;
  const int s = seq_of_row(a.cu_q, a.batch, tq);
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const bool valid = col < G && tq - sq.q0 < sq.nq;
  const int hh = h * G + (col < G ? col : 0);
  const int pos = sq.nk - sq.nq + (tq - sq.q0);
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  const int32_t* list = a.lists + ((size_t)tq * a.hkv + h) * a.topk;

  const float sl2 = a.scale_log2;
  bf16x8 bq[8];
  if (math)
    load_q_operand<false>(bq, reinterpret_cast<const char*>(a.q) + ((size_t)tq * a.hq + hh) * kD * 2, hf);

  const int per = (a.topk + a.splits - 1) / a.splits;
  const int slot0 = split * per, slot1 = min(a.topk, slot0 + per);
  if (tid < 64) visit_list(list, a.topk, slot0, slot1, nb, a.causal, pos, vis, &n_vis);
  // every load so far (Q rows, list, sequence bounds) completes here, before any K/V load is
  // issued: the compiler then has no load of its own pending inside the loop, where a wait of
  // its would also cover the K/V loads in flight
  if (math) hold_q(bq);
  wait_vm<0>();
  __syncthreads();
  const int nv = n_vis;

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(a.v);
  const uint32_t kv_row = (uint32_t)a.hkv * kD;
  const size_t kv_head = (size_t)sq.k0 * a.hkv + h;     // row of key 0 of the sequence, head h
  auto dma = [&](int j) {
    const int u0 = vis[j] * kBlock;
    const size_t off = (kv_head + (size_t)u0 * a.hkv) * kD;
    dma_rows<false>(L[j & 1].k, kp + off, kv_row, sq.nk - u0);
    dma_rows<true>(L[j & 1].vt, vp + off, kv_row, sq.nk - u0);
  };

  const float ninf = -__builtin_inff();
  // c_run: reference max in scaled (log2) units; l_run: this lane's share of the row sum
  float c_run = ninf, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  if (nv > 0) dma(0);
  for (int j = 0; j < nv; ++j) {
    wait_vm<0>();            // this thread's loads of block j landed
    __syncthreads();         // ... everyone's; step j - 1 is done, its buffer free
    if (j + 1 < nv) dma(j + 1);
    if (math) {
      const KVLds& B = L[j & 1];
      const int u0 = vis[j] * kBlock;
      f32x16 sc[2];
      qk_half(B.k, bq, sc, kt0, col, hf);
      int kmax = min(127, sq.nk - u0 - 1);
      if (a.causal) kmax = min(kmax, pos - u0);
      const float mb = mask_max_half(sc, kt0, kmax, __any(kmax < kt0 * 32 + 63), hf);
      const float mbs = mb * sl2;                        // -inf stays -inf (sl2 > 0)
      const bool grow = mbs > c_run + 8.f;
      if (__any(grow)) {
        const float c_new = grow ? mbs : c_run;
        const float alpha = grow ? (c_run > ninf ? __builtin_amdgcn_exp2f(c_run - c_new) : 0.f) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        c_run = c_new;
      }
      u32x4 pk[2][2];
      l_run += exp_pack_half(sc, sl2, c_run > ninf ? c_run : 0.f, pk);
      pv_half_tr(B.vt, pk, oacc, kt0, lane);
    }
  }
  l_run += shfl_xor_f(l_run, 32);            // the row's sum over the wave's keys

  if (a.splits > 1 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0)
    a.counters[0] = a.total_q * a.hkv * a.splits;
  // merge the key halves: wave 1 hands its (max, sum, output) to wave 0 through LDS (no load
  // is in flight: the last step issues none)
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&L[0]);          // [4 dt][4][64 lanes][4]
  float* xc = xo + 4 * 4 * 64 * 4;                      // [64 lanes] max, then sum
  if (wave == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 w = {oacc[dt][4 * q], oacc[dt][4 * q + 1], oacc[dt][4 * q + 2], oacc[dt][4 * q + 3]};
        *reinterpret_cast<f32x4*>(xo + ((dt * 4 + q) * 64 + lane) * 4) = w;
      }
    xc[lane] = c_run;
    xc[64 + lane] = l_run;
  }
  __syncthreads();
  if (wave != 0 || !valid) return;
  const float c1 = xc[lane], l1 = xc[64 + lane];
  const float cm = fmaxf(c_run, c1);
  const float w0 = c_run > ninf ? __builtin_amdgcn_exp2f(c_run - cm) : 0.f;
  const float w1 = c1 > ninf ? __builtin_amdgcn_exp2f(c1 - cm) : 0.f;
  const float l = w0 * l_run + w1 * l1;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(xo + ((dt * 4 + q) * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][4 * q + i] = w0 * oacc[dt][4 * q + i] + w1 * x[i];
    }
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const float lse_v = any ? (cm + log2f(l)) * 0.69314718055994531f : ninf;
  const int g = hh - h * G;
  if (a.splits == 1) {
    store_o_row(a.o + ((size_t)tq * a.hq + hh) * kD, oacc, inv, hf);
    if (hf == 0 && a.lse) a.lse[(size_t)tq * a.hq + hh] = lse_v;
  } else {
    const size_t pe = ((size_t)tq * a.hkv + h) * a.splits + split;
    store_o_part(a.part_o, pe * G + g, oacc, inv, hf);
    if (hf == 0) {
      a.part_lse[pe * G + g] = lse_v;
      a.part_l[pe * G + g] = 1.f;           // the partial output is already normalised
      if (g == 0) a.cmap[pe] = (int)pe;
    }
  }
}

// Per-tile lists, bf16: the 128 rows of one (Q tile, head) on 8 waves. Wave w takes rows
// 32*(w%4) .. +31 and keys 64*(w/4) .. +63 of every listed block, with its own running max,
// sum and output; the two key halves of a row are merged once at the end. K and V are
// double-buffered in LDS (128 KiB): at the top of step j the workgroup waits for block j,
// crosses its one barrier of the step, and issues block j+1 by direct-to-LDS loads, which then
// have a whole step to land. The two waves sharing a SIMD overlap one's softmax with the
// other's MFMAs. The running max is raised only when a block's max exceeds it by more than
// 2^8 in probability (the output is rescaled then); otherwise the probabilities are taken
// against the old max, which changes no result beyond rounding.
struct KVLds2 {
  u32x4 k[2][128 * 16];
  u32x4 v[2][128 * 16];
};

__global__ __launch_bounds__(512, 1) void attn_qt_kernel(QArgs a) {
  __shared__ KVLds2 L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int rg = wave & 3, kh = wave >> 2, kt0 = 2 * kh;
  const int r = rg * 32 + col;

  int tile, hh;
  xcd_tile_head(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x, gridDim.y, &tile, &hh);
  const int h = hh / (a.hq / a.hkv);
  const int s = blockIdx.z;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  if (tile * a.list_q >= sq.nq) return;
  const int il = tile * a.list_q + r;
  const bool valid = r < a.list_q && il < sq.nq;
  const int t = sq.q0 + (valid ? il : 0);
  const int32_t* list = a.lists + (((size_t)s * a.tiles_max + tile) * a.hkv + h) * a.topk;
  const int pos = sq.nk - sq.nq + (t - sq.q0);
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  const int pos_max = sq.nk - sq.nq + min(tile * a.list_q + a.list_q - 1, sq.nq - 1);

  int nv;
  const int vis_lane = visit_list_lanes(list, a.topk, nb, a.causal, pos_max, &nv);
  auto vis = [&](int j) { return __builtin_amdgcn_readlane(vis_lane, j); };

  const float sl2 = a.scale_log2;
  bf16x8 bq[8];
  load_q_operand<false>(bq, reinterpret_cast<const char*>(a.q) + ((size_t)t * a.hq + hh) * kD * 2, hf);

  // K/V transfers: waves 0-3 load K rows, waves 4-7 V rows (dma_rows layouts); thread u of
  // its half issues 8 loads, load p reading row 16p + u/16. A full block's addresses are the
  // block base (uniform), p times 16 rows (uniform) and one of two per-thread offsets.
  const char* kvb = reinterpret_cast<const char*>(tid < 256 ? a.k : a.v);
  const uint32_t row_bytes = (uint32_t)a.hkv * kD * 2;
  const size_t head_off = ((size_t)sq.k0 * a.hkv + h) * kD * 2;
  const int u = tid & 255, row0 = u >> 4, slot = u & 15;
  const int half_wave = __builtin_amdgcn_readfirstlane((tid & 255) >> 6);
  const bool is_v = tid >= 256;
  uint32_t col_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int f = is_v ? swz_v(row0) : ((row0 & 3) | (par << 2) | (((row0 >> 2) & 1) << 3));
    col_off[par] = (uint32_t)row0 * row_bytes + (uint32_t)((slot ^ f) * 16);
  }
  auto dma = [&](int j, bool v_part) {
    const int u0 = vis(j) * kBlock;
    const int nk_rel = sq.nk - u0;
    u32x4* dst = v_part ? L.v[j & 1] : L.k[j & 1];
    if (nk_rel >= kBlock) {
      const char* src = kvb + head_off + (size_t)u0 * row_bytes;
#pragma unroll
      for (int p = 0; p < 8; ++p)
        lds_dma16(src + p * 16 * row_bytes + col_off[p & 1], dst + p * 256 + half_wave * 64);
    } else {
      const uint16_t* base = reinterpret_cast<const uint16_t*>(kvb + head_off + (size_t)u0 * row_bytes);
      if (v_part) dma_rows_t<true>(dst, base, row_bytes / 2, nk_rel, u);
      else dma_rows_t<false>(dst, base, row_bytes / 2, nk_rel, u);
    }
  };
  auto dma_k = [&](int j) { if (!is_v) dma(j, false); };
  auto dma_v = [&](int j) { if (is_v) dma(j, true); };

  const float ninf = -__builtin_inff();
  // c_run: reference max in scaled (log2) units; l_run: this lane's share of the row sum
  float c_run = ninf, l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  if (nv > 0) {
    dma_k(0);
    dma_v(0);
  }
  for (int j = 0; j < nv; ++j) {
    wait_vm<0>();                            // this thread's K(j) and V(j) landed
    hold_q(bq);
    __syncthreads();                         // ... everyone's; step j-1 done by every wave
    const int u0 = vis(j) * kBlock;
    if (j + 1 < nv) {
      dma_k(j + 1);
      dma_v(j + 1);
    }
    f32x16 sc[2];
    qk_half(L.k[j & 1], bq, sc, kt0, col, hf);
    int kmax = min(127, sq.nk - u0 - 1);
    if (a.causal) kmax = min(kmax, pos - u0);
    const float mb = mask_max_half(sc, kt0, kmax, __any(kmax < kt0 * 32 + 63), hf);
    // the reference max is raised only when the block's max exceeds it by more than 2^8
    const float mbs = mb * sl2;                        // -inf stays -inf (sl2 > 0)
    const bool grow = mbs > c_run + 8.f;
    if (__any(grow)) {
      const float c_new = grow ? mbs : c_run;
      const float alpha = grow ? (c_run > ninf ? __builtin_amdgcn_exp2f(c_run - c_new) : 0.f) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      c_run = c_new;
    }
    u32x4 pk[2][2];
    l_run += exp_pack_half(sc, sl2, c_run > ninf ? c_run : 0.f, pk);
    pv_half_tr(L.v[j & 1], pk, oacc, kt0, lane);
  }

  l_run += shfl_xor_f(l_run, 32);            // the row's sum over the wave's keys

  // merge the key halves: waves 4-7 hand their (max, sum, output) to waves 0-3 through LDS
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&L);             // [4 rg][4 dt][4][64 lanes][4]
  float* xc = xo + 4 * 4 * 4 * 64 * 4;                  // [4 rg][64 lanes] max, then sum
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 w = {oacc[dt][4 * q], oacc[dt][4 * q + 1], oacc[dt][4 * q + 2], oacc[dt][4 * q + 3]};
        *reinterpret_cast<f32x4*>(xo + (((rg * 4 + dt) * 4 + q) * 64 + lane) * 4) = w;
      }
    xc[rg * 64 + lane] = c_run;
    xc[256 + rg * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1 || !valid) return;
  const float c1 = xc[rg * 64 + lane], l1 = xc[256 + rg * 64 + lane];
  const float cm = fmaxf(c_run, c1);
  const float w0 = c_run > ninf ? __builtin_amdgcn_exp2f(c_run - cm) : 0.f;
  const float w1 = c1 > ninf ? __builtin_amdgcn_exp2f(c1 - cm) : 0.f;
  const float l = w0 * l_run + w1 * l1;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(xo + (((rg * 4 + dt) * 4 + q) * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][4 * q + i] = w0 * oacc[dt][4 * q + i] + w1 * x[i];
    }
  const bool any = l > 0.f;
  store_o_row(a.o + ((size_t)t * a.hq + hh) * kD, oacc, any ? 1.f / l : 0.f, hf);
  if (hf == 0 && a.lse) a.lse[(size_t)t * a.hq + hh] = any ? (cm + log2f(l)) * 0.69314718055994531f : ninf;
}

hipError_t launch_qd_g(const QArgs& a, int group, dim3 grid, hipStream_t st) {
  dim3 blk(256);
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_qd_kernel<1>, grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL(attn_qd_kernel<2>, grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL(attn_qd_kernel<4>, grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL(attn_qd_kernel<8>, grid, blk, 0, st, a); break;
    default: hipLaunchKernelGGL(attn_qd_kernel<16>, grid, blk, 0, st, a); break;
  }
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_q_g(const QArgs& a, int group, dim3 grid, hipStream_t st) {
  dim3 blk(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((attn_q_kernel<FP8, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_q_kernel<FP8, 2>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_q_kernel<FP8, 4>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_q_kernel<FP8, 8>), grid, blk, 0, st, a); break;
    default: hipLaunchKernelGGL((attn_q_kernel<FP8, 16>), grid, blk, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_q(const msa_shape& s, const Geometry& g, const Layout& L,
                         const void* q, const void* k, const void* v, const float* descale,
                         float scale, const int32_t* lists, const int32_t* cu_q,
                         const int32_t* cu_k, char* ws, void* o, float* lse, hipStream_t st) {
  QArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.descale = descale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.lists = lists;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.o = reinterpret_cast<uint16_t*>(o);
  a.lse = lse;
  a.counters = g.splits > 1 ? reinterpret_cast<int32_t*>(ws + L.counters) : nullptr;
  a.cmap = g.splits > 1 ? reinterpret_cast<int32_t*>(ws + L.cmap) : nullptr;
  a.part_lse = g.splits > 1 ? reinterpret_cast<float*>(ws + L.part_lse) : nullptr;
  a.part_l = g.splits > 1 ? reinterpret_cast<float*>(ws + L.part_l) : nullptr;
  a.part_o = g.splits > 1 ? reinterpret_cast<uint16_t*>(ws + L.part_o) : nullptr;
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.batch = s.batch;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.topk = s.topk;
  a.list_q = s.list_q;
  a.tiles_max = (int)g.tiles_max;
  a.causal = s.causal;
  a.splits = g.splits;
  dim3 grid;
  if (s.list_q > 1) {
    if (g.tiles_max == 0) return hipSuccess;
    grid = dim3((unsigned)g.tiles_max, s.hq, s.batch);
    if (s.dtype == MSA_BF16) {
      hipLaunchKernelGGL(attn_qt_kernel, grid, dim3(512), 0, st, a);
      return hipGetLastError();
    }
  } else {
    if (s.total_q == 0) return hipSuccess;
    grid = dim3((unsigned)s.total_q, s.hkv, g.splits);
    if (s.dtype == MSA_BF16) return launch_qd_g(a, g.group, grid, st);
  }
  return launch_q_g<true>(a, g.group, grid, st);
}

}  // namespace msa
