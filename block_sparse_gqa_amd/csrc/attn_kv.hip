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
// workgroups automatically). A workgroup of eight waves walks its slice bucket by bucket: it
// stages the bucket's K and V^T in LDS once, then processes tiles of 256 rows = 256/G entries
// x G heads, 32 rows per wave, two waves per SIMD. Each entry's G x D partial lands in rows
// e*G .. e*G+G-1 of the partial buffer, so a wave's 32 output rows are one contiguous 8 KiB
// range; they are written through a per-wave LDS buffer so that every store instruction
// covers 1 KiB of consecutive bytes.
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
  const int32_t* entry_bucket;
  float* part_lse;
  float* part_l;
  uint16_t* part_o;
  uint16_t* dummy;
  int total_q, total_k, max_q, max_k;
  int hq, hkv, nb_max, wr, n_r, n_buckets, n_wg, causal;
};

// --------------------------------------------------------------------------------------
// Per-wave tile step. The MFMA pipe and the VALU of a SIMD run concurrently when MFMAs and
// independent VALU work alternate in the instruction stream, so each tile is done in two
// interleaved phases:
//   phase A, step st: 4 MFMAs of QK^T(j) (d-step st)  | O(j-1): bf16 packing into the wave's
//                                                      |   LDS buffer (steps 0-3), coalesced
//                                                      |   read-back and stores (steps 4-7)
//   row max of S(j)
//   phase B, step s:  4 MFMAs of PV(j) (key-step s)    | exp2 + packing of key-step s+1
// LDS operands are double-buffered over the 16 steps; everything else stays in VGPRs.

// K operands (A) of d-step st for the 4 key tiles.
__device__ __forceinline__ void k_frags(const KVLds& L, bf16x8 a[4], int st, int rp, int sw,
                                        int hf) {
  const int cc = (2 * st + hf) ^ sw;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) a[kt] = as_bf16x8(L.k[(kt * 32 + rp) * 16 + cc]);
}

// V^T operands (A) of key-step s for the 4 output-dim tiles.
__device__ __forceinline__ void v_frags(const KVLds& L, bf16x8 a[4], int s, int rp, int sw,
                                        int hf) {
  const int cc = (4 * (s >> 1) + 2 * hf + (s & 1)) ^ sw;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) a[dt] = as_bf16x8(L.vt[(dt * 32 + rp) * 16 + cc]);
}

// exp2 of the 8 scores of key-step s, packed to bf16 into pk; their sum is added to l. The
// sum is taken over the bf16-rounded weights (one bf16 dot product per pair), the exact
// weights the PV product uses.
__device__ __forceinline__ float exp_step(const f32x16 sc[4], int s, float sl2, float c,
                                          u32x4& pk, float l) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const int kt = s >> 1, base = 8 * (s & 1);
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = __builtin_amdgcn_exp2f(fmaf(sc[kt][base + 2 * i], sl2, -c));
    const float x1 = __builtin_amdgcn_exp2f(fmaf(sc[kt][base + 2 * i + 1], sl2, -c));
    // (the packed pair is taken as a value: a bit_cast of the vector element reference pk[i]
    // has been compiled to read element 0 for every i)
    const uint32_t pw = pack_bf16x2(x0, x1);
    pk[i] = pw;
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw), ones, l, false);
  }
  return l;
}

// Output staging: the wave's 32 rows x 256 B, 16-byte chunk c of row R at R*16 + (c ^ (R%16)).
// Lane (col, hf) deposits dims 32*dt + 16*hf .. +15 of row col (chunks 4dt+2hf, +1).
template <bool FP8>
__device__ __forceinline__ void stage_o(u32x4* buf, const f32x16& o, int dt, float mul,
                                        int col, int hf) {
  // opaque copies: the addresses are recomputed here instead of being held (or spilled)
  // across the caller's loop
  asm volatile("" : "+v"(col), "+v"(hf));
  const int x = (2 * hf) ^ (col & 15);   // c ^ (col % 16) == (4dt + h2) ^ x
  u32x4* const row = buf + col * 16;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (FP8)   // the V descale; bf16 stores the accumulator as it is
        w[i] = pack_bf16x2(o[8 * h2 + 2 * i] * mul, o[8 * h2 + 2 * i + 1] * mul);
      else
        w[i] = pack_bf16x2(o[8 * h2 + 2 * i], o[8 * h2 + 2 * i + 1]);
    }
    row[(4 * dt + h2) ^ x] = w;
  }
}

// Read-back i (0..7): lane l takes chunk l%16 of row R = 4i + l/16, so the 64 lanes hold
// 1 KiB of consecutive output bytes. With R % 16 = 4 (i % 4) + l/16 the slot is
// (l%16) ^ (l/16) ^ 4 (i % 4): the lane's address for read-back i is ub[i % 4] + 256 (i / 4).
__device__ __forceinline__ void unstage_bases(int lane, int ub[4]) {
  asm volatile("" : "+v"(lane));
  const int lq = lane >> 4, x = (lane & 15) ^ lq;
#pragma unroll
  for (int j = 0; j < 4; ++j) ub[j] = (4 * j + lq) * 16 + (x ^ (4 * j));
}

// Q rows of the wave's next tile into its staging buffer with direct-to-LDS loads. `rowidx`
// is the lane's own Q row index (query * hq + head). A row is RB = 128 * EB bytes = RB / 16
// chunks; load i brings rows (64 / CPR) i .. +(64 / CPR - 1), lane l fetching the chunk that
// belongs in slot l % CPR of its row (chunk c of row R sits in slot c ^ (R % CPR)), so each
// load reads 1 KiB of whole rows.
template <bool FP8, int G>
__device__ __forceinline__ void dma_q(u32x4* buf, const void* q, int rowidx, int lane) {
  constexpr int RB = FP8 ? 128 : 256;    // bytes per Q row
  constexpr int CPR = RB / 16;           // chunks per row
  constexpr int RPL = 64 / CPR;          // rows per load
  asm volatile("" : "+v"(lane));
  const char* qb = reinterpret_cast<const char*>(q);
  const int lr = lane / CPR, lc = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPL; ++i) {
    const int R = RPL * i + lr;
    int src_row;
    if constexpr (G >= RPL) {
      // the load's rows are consecutive heads of one query: Q rows row0 .. row0 + RPL - 1,
      // row0 being the row index held by the lane of row RPL * i
      src_row = __builtin_amdgcn_readlane(rowidx, RPL * i) + lr;
    } else {
      src_row = __shfl(rowidx, R);
    }
    const int c = lc ^ (R % CPR);
    __builtin_amdgcn_global_load_lds(
        qb + (size_t)src_row * RB + c * 16,
        (__attribute__((address_space(3))) void*)(buf + 64 * i), 16, 0, 0);
  }
}

// B operand of S^T from the staging buffer: elements 16*st + 8*hf .. +7 of the lane's row.
template <bool FP8>
__device__ __forceinline__ void read_q(const u32x4* buf, bf16x8 bq[8], int col, int hf) {
  asm volatile("" : "+v"(col), "+v"(hf));
  if constexpr (!FP8) {
    const int x = hf ^ (col & 15);          // (2st + hf) ^ (col % 16) == 2st ^ x
    const u32x4* const row = buf + col * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) bq[st] = as_bf16x8(row[(2 * st) ^ x]);
  } else {
    const u32x2* const row = reinterpret_cast<const u32x2*>(buf + col * 8);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x2 v = row[2 * (st ^ (col & 7)) + hf];
      const u32x2 lo = fp8x4_to_bf16x4(v[0]);
      const u32x2 hi = fp8x4_to_bf16x4(v[1]);
      bq[st] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  }
}

// s_waitcnt vmcnt(0): direct-to-LDS loads are not tracked by the compiler's own waits.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scheduling request for one phase-A step: the first MFMA, the 4 LDS reads of the next
// step's operands, then MFMAs each followed by NVALU VALU instructions.
#define MSA_INTERLEAVE(ID, NVALU)                                 \
  do {                                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);           \
    __builtin_amdgcn_sched_group_barrier(0x100, 4, ID);           \
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, ID);       \
    _Pragma("unroll") for (int q_ = 0; q_ < 3; ++q_) {            \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);         \
      __builtin_amdgcn_sched_group_barrier(0x002, NVALU, ID);     \
    }                                                             \
    __builtin_amdgcn_sched_barrier(0);                            \
  } while (0)

template <bool FP8, int G>
__global__ __launch_bounds__(512, 1) void attn_kv_kernel(KvArgs a) {
  constexpr int MQ = 256 / G;          // entries per tile
  constexpr int EB = FP8 ? 1 : 2;      // bytes per Q/K/V element
  __shared__ KVLds L;
  __shared__ u32x4 obuf_all[8][32 * 16];

  const int E = a.counters[0];
  if (E == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int r = wave * 32 + col;       // row of the tile
  const int rent = r / G, g = r % G;
  const int rp = rowperm(col), sw = swz(rp);
  u32x4* const obuf = obuf_all[wave];

  float sl2 = a.scale_log2, dv = 1.f;
  if constexpr (FP8) {
    sl2 *= a.descale[0] * a.descale[1];
    dv = a.descale[2];
  }
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const uint32_t kv_row = (uint32_t)a.hkv * kD;    // elements between consecutive keys
  const int last = E - 1;
  // Sinks for the stores of padding rows (contents never read).
  uint16_t* const o_sink = a.dummy + lane * 8;
  float* const lse_sink = reinterpret_cast<float*>(a.dummy + 64 * 8) + lane;
  float* const l_sink = reinterpret_cast<float*>(a.dummy + 128 * 8) + lane;

  // Phases (sequence, group, query range) in entry order; this workgroup's share of each.
  const int n_phase = a.n_buckets / a.nb_max;
  for (int ph = 0; ph < n_phase; ++ph) {
  const int p_begin = a.offsets[(size_t)ph * a.nb_max * a.wr];
  const int p_end = (ph + 1 < n_phase) ? a.offsets[(size_t)(ph + 1) * a.nb_max * a.wr] : E;
  const int e_begin = p_begin + (int)((int64_t)(p_end - p_begin) * blockIdx.x / a.n_wg);
  const int e_end = p_begin + (int)((int64_t)(p_end - p_begin) * (blockIdx.x + 1) / a.n_wg);
  int cur = e_begin;
  while (cur < e_end) {
    const int bk = a.entry_bucket[cur];
    if ((unsigned)bk >= (unsigned)a.n_buckets) break;   // never for a planned workspace
    const int bend = (bk + 1 < a.n_buckets) ? a.offsets[(size_t)(bk + 1) * a.wr] : E;
    const int run_end = min(e_end, bend);
    const int b = bk % a.nb_max;
    const int h = (bk / (a.nb_max * a.n_r)) % a.hkv;
    const int s = bk / (a.nb_max * a.n_r * a.hkv);
    const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
    const int u0 = b * kBlock;
    const int nk_rel = sq.nk - u0;

    __syncthreads();   // LDS of the previous block no longer read
    if (tid < 256)
      stage_kv<FP8>(L, kb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB,
                    vb + ((size_t)(sq.k0 + u0) * a.hkv + h) * kD * EB, kv_row, nk_rel);
    __syncthreads();

    auto qidx = [&](int e, int tv) { return (e < run_end ? tv : sq.q0) * a.hq + h * G + g; };

    int e0 = cur + rent, e1 = e0 + MQ;
    int t0v = a.entry_q[min(e0, last)];
    int t1v = a.entry_q[min(e1, last)];
    bf16x8 bq[8];
    int ub[4];
    unstage_bases(lane, ub);
    dma_q<FP8, G>(obuf, a.q, qidx(e0, t0v), lane);
    // LDS operands, double-buffered over the 16 steps of a tile (8 K steps, then 8 V steps):
    // step i reads fr[i & 1] while the reads of step i + 1 are in flight.
    bf16x8 fr[2][4];
    k_frags(L, fr[0], 0, rp, sw, hf);
    // output of the previous tile: none yet (its rows all count as padding)
    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    float o_l = 0.f, o_lse = 0.f;
    // stores of the previous tile: rows 4i + lane/16 of the wave at o_base + 4i rows, valid
    // while 4i < o_nv (none yet)
    uint16_t* o_base = o_sink;
    int o_nv = 0;
    float* lse_ptr = lse_sink;
    float* l_ptr = l_sink;

    for (int tile0 = cur; tile0 < run_end; tile0 += MQ) {
      const int e2 = e1 + MQ;
      const int t2v = a.entry_q[min(e2, last)];
      int kmax = min(127, nk_rel - 1);
      if (a.causal) kmax = min(kmax, sq.nk - sq.nq + (t0v - sq.q0) - u0);
      const bool need_mask = __any(kmax < 127);
      const bool valid = e0 < run_end;
      wait_vm0();               // this tile's Q rows have landed in the staging buffer
      read_q<FP8>(obuf, bq, col, hf);

      // ---- phase A: QK^T(j) | O(j-1) through LDS to memory
      f32x16 sc[4];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st < 7) k_frags(L, fr[(st + 1) & 1], st + 1, rp, sw, hf);
        else v_frags(L, fr[0], 0, rp, sw, hf);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sc[kt] = mfma32(fr[st & 1][kt], bq[st], st == 0 ? f32x16{} : sc[kt]);
        if (st < 4) {
          stage_o<FP8>(obuf, oacc[st], st, dv, col, hf);
        } else {
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const int i = 2 * (st - 4) + i2;
            const u32x4 w = obuf[ub[i & 3] + 256 * (i >> 2)];
            // streaming store: the partials are read once, by the combine kernel
            __builtin_nontemporal_store(
                w, reinterpret_cast<u32x4*>(4 * i < o_nv ? o_base + i * 4 * kD : o_sink));
          }
          if (st == 7) {
            *lse_ptr = o_lse;
            *l_ptr = o_l;
          }
        }
        MSA_INTERLEAVE(1, 6);
      }
      // Q of the next tile into the staging buffer, whose read-back for the stores above is
      // complete
      dma_q<FP8, G>(obuf, a.q, qidx(e1, t1v), lane);
      // ---- row max of S(j)
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sc[kt][i] = (kt * 32 + 16 * hf + i <= kmax) ? sc[kt][i] : -__builtin_inff();
      }
      float m = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, sc[kt][i]);
      m = fmaxf(m, shfl_xor_f(m, 32));
      const bool any = m > -__builtin_inff();
      const float c = any ? m * sl2 : 0.f;
      // ---- phase B: PV(j) | exp of the next key-step
      u32x4 pk[8];
      float l = exp_step(sc, 0, sl2, c, pk[0], 0.f);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        // the last step fetches the first K operands of the next tile (discarded after the
        // run's last tile)
        if (st < 7) v_frags(L, fr[(st + 1) & 1], st + 1, rp, sw, hf);
        else k_frags(L, fr[0], 0, rp, sw, hf);
        const bf16x8 bp = as_bf16x8(pk[st]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          oacc[dt] = mfma32(fr[st & 1][dt], bp, st == 0 ? f32x16{} : oacc[dt]);
        if (st + 1 < 8) l = exp_step(sc, st + 1, sl2, c, pk[st + 1], l);
        MSA_INTERLEAVE(2, 7);
      }
      l += shfl_xor_f(l, 32);
      // the output of tile j is stored during the next tile's phase A
      o_l = any ? l : 0.f;
      o_lse = any ? (c + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
      {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        o_base = a.part_o + ((size_t)tile0 * G + wave * 32 + (ln >> 4)) * kD + (ln & 15) * 8;
        o_nv = (run_end - tile0) * G - wave * 32 - (ln >> 4);
      }
      lse_ptr = valid ? a.part_lse + (size_t)e0 * G + g : lse_sink;
      l_ptr = valid ? a.part_l + (size_t)e0 * G + g : l_sink;
      e0 = e1;
      e1 = e2;
      t0v = t1v;
      t1v = t2v;
    }
    // output of the run's last tile (after the last, unused, Q load into the buffer)
    wait_vm0();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) stage_o<FP8>(obuf, oacc[dt], dt, dv, col, hf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 w = obuf[ub[i & 3] + 256 * (i >> 2)];
      __builtin_nontemporal_store(
          w, reinterpret_cast<u32x4*>(4 * i < o_nv ? o_base + i * 4 * kD : o_sink));
    }
    *lse_ptr = o_lse;
    *l_ptr = o_l;
    cur = run_end;
  }
  }
}

template <bool FP8>
hipError_t launch_kv_g(const KvArgs& a, int group, int n_wg, hipStream_t st) {
  dim3 grid(n_wg), blk(512);
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
  a.part_l = reinterpret_cast<float*>(ws + L.part_l);
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
  const int n_wg = device_cu_count();   // one workgroup (eight waves) per CU
  a.n_wg = n_wg;
  return s.dtype == MSA_FP8_E4M3 ? launch_kv_g<true>(a, g.group, n_wg, st)
                                 : launch_kv_g<false>(a, g.group, n_wg, st);
}

}  // namespace msa
