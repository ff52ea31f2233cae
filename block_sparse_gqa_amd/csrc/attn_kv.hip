// KV-outer (KV-stationary) main attention kernel.
//
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell" (summary and section 2): each
// selected KV block is loaded once in the outer loop and every query that chose it is
// gathered in the inner loop; a work unit owns a single block, so there is one softmax step
// and no rescaling; partial outputs are written contiguously in work order. The GQA heads of
// one query form a contiguous box of Q rows, gathered with one index read per query-group.
//
// The entry list built by the plan kernels is cut into equal contiguous slices, one per
// persistent workgroup (deterministic, no atomics; heavy blocks are split between
// workgroups automatically). A workgroup walks its slice bucket by bucket: it stages the
// bucket's K and V^T in LDS once, then processes tiles of 128 rows = 128/G entries x G heads
// with four waves of 32 rows. Each entry's G x D partial lands in rows e*G .. e*G+G-1 of the
// partial buffer, so a tile's stores form one contiguous 32 KiB range.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14); expcnt and lgkmcnt left at their maxima (no wait).
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm27 = 0x0F70 | (27 & 15) | ((27 >> 4) << 14);

struct KvArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* descale;
  float scale_log2;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* counters;
  const int32_t* offsets;
  const int32_t* entry_q;
  const int32_t* entry_bucket;
  float* part_lse;
  uint16_t* part_o;
  uint16_t* dummy;
  int total_q, total_k, max_q, max_k;
  int hq, hkv, nb_max, wr, n_r, n_buckets, n_wg, causal;
};

template <bool FP8, int G>
__global__ __launch_bounds__(256, 2) void attn_kv_kernel(KvArgs a) {
  constexpr int MQ = 128 / G;          // entries per tile
  constexpr int EB = FP8 ? 1 : 2;      // bytes per Q/K/V element
  __shared__ KVLds L;

  const int E = a.counters[0];
  // Chunks of kChunkTiles tiles go round-robin to the workgroups, so that at any time the
  // whole grid works on one window of the entry order (one query range of one group: its Q
  // rows are then re-read from cache). Workgroup ids are dispatched round-robin over the 8
  // XCDs; renumbering them XCD-major gives each XCD runs of consecutive chunks, which share
  // K/V blocks in that XCD's L2.
  const int n_xcd = 8;
  const int per_xcd = a.n_wg / n_xcd;
  const int lw = (int)(blockIdx.x % n_xcd) * per_xcd + (int)(blockIdx.x / n_xcd);
  constexpr int CHUNK = kChunkTiles * MQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int r = wave * 32 + col;       // row of the tile
  const int rent = r / G, g = r % G;

  float sl2 = a.scale_log2, dv = 1.f;
  if constexpr (FP8) {
    sl2 *= a.descale[0] * a.descale[1];
    dv = a.descale[2];
  }
  const char* qb = reinterpret_cast<const char*>(a.q);
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const uint32_t kv_row = (uint32_t)a.hkv * kD;    // elements between consecutive keys

  int staged = -1;                     // bucket whose K/V sit in LDS
  // Packed output of the last tile, stored during the next tile. Until a first tile exists
  // it points at the sink.
  u32x4 wout[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) wout[j] = u32x4{0u, 0u, 0u, 0u};
  uint16_t* pend_o = a.dummy + (size_t)r * kD;
  float* pend_lse_ptr = reinterpret_cast<float*>(a.dummy + 128 * kD) + r;
  float pend_lse = 0.f;
  for (int64_t c0 = (int64_t)lw * CHUNK; c0 < E; c0 += (int64_t)a.n_wg * CHUNK) {
  const int c1 = (int)min<int64_t>(E, c0 + CHUNK);
  int cur = (int)c0;
  while (cur < c1) {
    const int bk = a.entry_bucket[cur];
    if ((unsigned)bk >= (unsigned)a.n_buckets) break;   // never for a planned workspace
    const int bend = (bk + 1 < a.n_buckets) ? a.offsets[(size_t)(bk + 1) * a.wr] : E;
    const int run_end = min(c1, bend);
    const int b = bk % a.nb_max;
    const int h = (bk / (a.nb_max * a.n_r)) % a.hkv;
    const int s = bk / (a.nb_max * a.n_r * a.hkv);
    const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
    const int u0 = b * kBlock;
    const int nk_rel = sq.nk - u0;
    const int kvkey = (s * a.hkv + h) * a.nb_max + b;

    if (kvkey != staged) {
      __syncthreads();   // LDS of the previous block no longer read
      stage_kv<FP8>(L, kb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB,
                    vb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB, kv_row, nk_rel);
      __syncthreads();
      staged = kvkey;
    }

    // Tile pipeline. Per tile, in issue order: the entry index of the tile three steps ahead
    // (1 load), the Q rows of the tile two steps ahead (8 loads), the QK^T MFMAs, the 9
    // stores of the previous tile's output (its registers are not reused before they are
    // read), softmax and PV. Every one of these memory operations is issued by every lane
    // (padding rows read a valid row and write to a sink), so the explicit wait at the end of
    // a tile is exact: the next tile's Q rows (loaded one tile earlier) must have arrived;
    // the 27 operations issued after them may stay in flight.
    const int last = E - 1;
    int e0 = cur + rent, e1 = e0 + MQ, e2 = e1 + MQ;
    int t0v = a.entry_q[min(e0, last)], t1v = a.entry_q[min(e1, last)];
    int t2v = a.entry_q[min(e2, last)];
    auto qrow = [&](int e, int tv) {
      return qb + ((size_t)(e < run_end ? tv : sq.q0) * a.hq + h * G + g) * kD * EB;
    };
    bf16x8 bq[8], bq1[8];
    load_q_operand<FP8>(bq, qrow(e0, t0v), hf);
    load_q_operand<FP8>(bq1, qrow(e1, t1v), hf);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    for (int tile0 = cur; tile0 < run_end; tile0 += MQ) {
      const int e3 = e2 + MQ;
      const int t3v = a.entry_q[min(e3, last)];
      bf16x8 bq2[8];
      load_q_operand<FP8>(bq2, qrow(e2, t2v), hf);

      f32x16 sacc[4];
      qk_block(L, bq, sacc, col, hf);
      store_packed_row(pend_o, wout, hf);
      *pend_lse_ptr = pend_lse;
      const int t = t0v;
      const bool valid = e0 < run_end;
      const int pos = sq.nk - sq.nq + (t - sq.q0);
      int kmax = min(127, nk_rel - 1);
      if (a.causal) kmax = min(kmax, pos - u0);
      const bool need_mask = __any(kmax < 127);
      const float m = mask_max(sacc, kmax, need_mask, hf);
      const bool any = m > -__builtin_inff();
      const float c = any ? m * sl2 : 0.f;
      u32x4 pk[4][2];
      const float l = exp_pack(sacc, sl2, c, pk);

      f32x16 oacc[4];
      pv_block<true>(L, pk, oacc, col, hf);

      pack_o_row(wout, oacc, any ? dv / l : 0.f);
      const size_t prow = valid ? (size_t)e0 * G + g : (size_t)r;
      pend_o = (valid ? a.part_o : a.dummy) + prow * kD;
      pend_lse_ptr = (valid ? a.part_lse : reinterpret_cast<float*>(a.dummy + 128 * kD)) + prow;
      pend_lse = any ? (c + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
      __builtin_amdgcn_s_waitcnt(kWaitVm27);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        bq[st] = bq1[st];
        bq1[st] = bq2[st];
      }
      e0 = e1;
      e1 = e2;
      e2 = e3;
      t0v = t1v;
      t1v = t2v;
      t2v = t3v;
    }
    cur = run_end;
  }
  }
  store_packed_row(pend_o, wout, hf);
  *pend_lse_ptr = pend_lse;
}

template <bool FP8>
hipError_t launch_kv_g(const KvArgs& a, int group, int n_wg, hipStream_t st) {
  dim3 grid(n_wg), blk(256);
  switch (group) {
    case 1: hipLaunchKernelGGL((attn_kv_kernel<FP8, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((attn_kv_kernel<FP8, 2>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((attn_kv_kernel<FP8, 4>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_kv_kernel<FP8, 8>), grid, blk, 0, st, a); break;
    default: hipLaunchKernelGGL((attn_kv_kernel<FP8, 16>), grid, blk, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_kv(const msa_shape& s, const Geometry& g, const Layout& L,
                          const void* q, const void* k, const void* v, const float* descale,
                          float scale, const int32_t* cu_q, const int32_t* cu_k, char* ws,
                          hipStream_t st) {
  KvArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.descale = descale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.counters = reinterpret_cast<const int32_t*>(ws + L.counters);
  a.offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  a.entry_q = reinterpret_cast<const int32_t*>(ws + L.entry_q);
  a.entry_bucket = reinterpret_cast<const int32_t*>(ws + L.entry_bucket);
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  a.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
  a.dummy = reinterpret_cast<uint16_t*>(ws + L.dummy);
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.nb_max = (int)g.nb_max;
  a.wr = (int)g.wr;
  a.n_r = (int)g.n_r;
  a.n_buckets = (int)g.n_buckets;
  a.causal = s.causal;
  if (g.n_words == 0) return hipSuccess;
  const int n_wg = 2 * ((device_cu_count() + 7) / 8) * 8;
  a.n_wg = n_wg;
  return s.dtype == MSA_FP8_E4M3 ? launch_kv_g<true>(a, g.group, n_wg, st)
                                 : launch_kv_g<false>(a, g.group, n_wg, st);
}

}  // namespace msa
