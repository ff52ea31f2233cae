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
  float* part_lse;
  uint16_t* part_o;
  int total_q, total_k, max_q, max_k;
  int hq, hkv, nb_max, w_max, n_buckets, n_wg, causal;
};

template <bool FP8, int G>
__global__ __launch_bounds__(256, 2) void attn_kv_kernel(KvArgs a) {
  constexpr int MQ = 128 / G;          // entries per tile
  constexpr int EB = FP8 ? 1 : 2;      // bytes per Q/K/V element
  __shared__ KVLds L;

  const int E = a.counters[0];
  const int64_t e_begin = (int64_t)E * blockIdx.x / a.n_wg;
  const int64_t e_end = (int64_t)E * (blockIdx.x + 1) / a.n_wg;
  if (e_begin >= e_end) return;

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

  int cur = (int)e_begin;
  while (cur < (int)e_end) {
    // bucket holding entry `cur`: the last bucket whose first entry is <= cur
    int lo = 0, hi = a.n_buckets - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[(size_t)mid * a.w_max] <= cur) lo = mid; else hi = mid - 1;
    }
    const int bk = lo;
    const int bend = (bk + 1 < a.n_buckets) ? a.offsets[(size_t)(bk + 1) * a.w_max] : E;
    const int run_end = min((int)e_end, bend);
    const int s = bk / (a.hkv * a.nb_max);
    const int h = (bk / a.nb_max) % a.hkv;
    const int b = bk % a.nb_max;
    const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
    const int u0 = b * kBlock;
    const int nk_rel = sq.nk - u0;

    __syncthreads();   // LDS of the previous bucket no longer read
    stage_kv<FP8>(L, kb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB,
                  vb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB, kv_row, nk_rel);
    __syncthreads();

    for (int t0 = cur; t0 < run_end; t0 += MQ) {
      const int ent = t0 + rent;
      const bool valid = ent < run_end;
      const int t = valid ? a.entry_q[ent] : sq.q0;
      bf16x8 bq[8];
      load_q_operand<FP8>(bq, qb + ((size_t)t * a.hq + h * G + g) * kD * EB, valid, hf);
      f32x16 sacc[4];
      qk_block(L, bq, sacc, col, hf);

      const int pos = sq.nk - sq.nq + (t - sq.q0);
      int kmax = min(127, nk_rel - 1);
      if (a.causal) kmax = min(kmax, pos - u0);
      const float m = scale_mask_max(sacc, sl2, kmax, hf);
      const bool any = m > -__builtin_inff();
      const float ms = any ? m : 0.f;
      const float l = exp_sum(sacc, ms);

      f32x16 oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
      pv_block(L, sacc, oacc, col, hf);

      if (valid) {
        const float inv = any ? dv / l : 0.f;
        const size_t prow = (size_t)ent * G + g;
        store_o_row(a.part_o + prow * kD, oacc, inv, hf);
        if (hf == 0)
          a.part_lse[prow] = any ? (ms + log2f(l)) * 0.69314718055994531f
                                 : -__builtin_inff();
      }
    }
    cur = run_end;
  }
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
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  a.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.nb_max = (int)g.nb_max;
  a.w_max = (int)g.w_max;
  a.n_buckets = (int)g.n_buckets;
  a.causal = s.causal;
  if (g.n_words == 0) return hipSuccess;
  const int n_wg = 2 * device_cu_count();
  a.n_wg = n_wg;
  return s.dtype == MSA_FP8_E4M3 ? launch_kv_g<true>(a, g.group, n_wg, st)
                                 : launch_kv_g<false>(a, g.group, n_wg, st);
}

}  // namespace msa
