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


// ======================================================================================
// bf16: tiles of XCD-local query ranges, K/V restaged asynchronously.
//
// The plan cuts the entries of every (sequence, group, 512-query range) phase into tiles of
// 256 / G entries of one bucket and writes one record per tile. Phase p belongs to XCD
// p % n_xcd (workgroup i runs on XCD i % n_xcd), whose n_share workgroups split the phase's
// tiles into contiguous shares; the Q rows of a phase (2 MiB for 16 heads) stay in that XCD's
// L2 while every block of the range re-reads them.
//
// K and V blocks go to LDS by direct loads into three rotating 32 KiB slots. When the next
// tile starts a new bucket, its K block is loaded at the start of the current tile into the
// free slot (the V slot of the previous bucket, released by the barrier that opened the
// current bucket) and its V block, after a barrier, into the K slot of the current bucket once
// every wave has finished QK^T; the next tile starts after one more barrier. V stays
// row-major and is read with the LDS transpose load. Output stores go through buffer
// descriptors whose record count covers the tile's real rows: stores of padding rows are
// dropped by the hardware range check.
//
// All direct-to-LDS loads are issued as inline assembly and ordered by the kernel's own waits
// (one vmcnt(0) at the start of each tile, then a barrier when the tile opens a bucket): the
// compiler, which cannot tell the destination slots apart, would otherwise wait for every
// outstanding load before each LDS read. Tile records are read one tile before they are
// decoded (their loads are covered by that same wait) and the entry queries of the next tile
// at the start of the current one.

struct KvTArgs {
  const void* q;
  const void* k;
  const void* v;
  float scale_log2;
  const int32_t* __restrict__ cu_q;
  const int32_t* __restrict__ cu_k;
  const int32_t* __restrict__ counters;
  const int32_t* __restrict__ entry_q;
  const int32_t* __restrict__ phase_base;
  const int2* __restrict__ recs;
  float* part_lse;
  float* part_l;
  uint16_t* part_o;
  int total_q, total_k, max_q, max_k;
  int hq, hkv, nb_max, n_r, n_phase, n_xcd, n_share, causal;
};

// 16 bytes per lane from global memory to LDS address m0 + 16 * lane (m0 wave-uniform).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
// The same from a wave-uniform base plus a 32-bit lane offset.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  const __attribute__((address_space(3))) char* l = (const __attribute__((address_space(3))) char*)p;
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
}

// A tile: entries [e0, e0 + n) of block b of phase p (n = 0: past the end of the stream).
struct TileD {
  int e0, n, b, p;
};

// A record read ahead: raw (first entry, block << 8 | n - 1) in vector registers and its
// phase (n_phase past the end of the stream).
struct TileRaw {
  int2 r;
  int p;
};

// The workgroup's tile stream: its share of every phase p = xcd, xcd + n_xcd, ... in order.
struct TileIt {
  int p, t, t_end;
};

__device__ __forceinline__ void it_enter(TileIt& it, const KvTArgs& a, int j) {
  while (it.p < a.n_phase) {
    const int pb0 = a.phase_base[it.p], pb1 = a.phase_base[it.p + 1];
    // n * n_share stays far below 2^31 (a phase holds at most 512 * 16 entries)
    const int n = pb1 - pb0;
    // The share taken rotates with the phase: the last share of a causal phase holds the
    // range's own blocks, whose tiles need the causal mask; rotating spreads them evenly.
    const int jj = (j + it.p / a.n_xcd) % a.n_share;
    it.t = pb0 + (int)((uint32_t)(n * jj) / (uint32_t)a.n_share);
    it.t_end = pb0 + (int)((uint32_t)(n * (jj + 1)) / (uint32_t)a.n_share);
    if (it.t < it.t_end) return;
    it.p += a.n_xcd;
  }
}

__device__ __forceinline__ TileRaw it_fetch(TileIt& it, const KvTArgs& a, int j) {
  TileRaw x;
  x.p = it.p;
  x.r = make_int2(0, 0);
  if (it.p >= a.n_phase) return x;
  int z = 0;
  asm volatile("" : "+v"(z));      // keeps the record in vector registers until decoded
  x.r = a.recs[it.t + z];
  if (++it.t == it.t_end) {
    it.p += a.n_xcd;
    it_enter(it, a, j);
  }
  return x;
}

__device__ __forceinline__ TileD it_decode(const TileRaw& x, TileIt& it, const KvTArgs& a, int E) {
  TileD d{0, 0, 0, x.p};
  if (x.p >= a.n_phase) return d;
  d.e0 = __builtin_amdgcn_readfirstlane(x.r.x);
  const int y = __builtin_amdgcn_readfirstlane(x.r.y);
  d.n = (y & 255) + 1;
  d.b = y >> 8;
  // a record inconsistent with the entry count ends the stream (never for a planned workspace)
  if (d.e0 < 0 || d.e0 > E - d.n || d.b >= a.nb_max) {
    it.p = a.n_phase;
    d.n = 0;
  }
  return d;
}

// K (layout of k_frags) or V (row-major, transposed reads) of one block into an LDS slot by
// the workgroup's 512 threads, 4 direct loads each: load p of wave w fills rows
// 32p + 4w .. +3, lane l fetching the chunk that belongs in its slot. Rows at or past nk_rel
// repeat the last key (their scores are masked).
template <bool V>
__device__ __forceinline__ void dma_block(u32x4* dst, const uint16_t* base, uint32_t row_stride,
                                          int nk_rel, int wave, int lane) {
  const int slot = lane & 15;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 32 * p + 4 * wave + (lane >> 4);
    const int f = V ? swz_v(row) : swz(row);
    const uint32_t r = (uint32_t)min(row, nk_rel - 1);
    dma16s(base, (r * row_stride + (uint32_t)((slot ^ f) * 8)) * 2,
           lds_addr(dst + p * 512 + wave * 64));
  }
}

// V^T operands (A) of key-step s (keys 32kt + 16hf + 8ks .. +7, kt = s/2, ks = s%2) for the
// 4 output-dim tiles, from the row-major V block by transpose loads; `vl` is the lane's
// element offset within the slot (see pv_block_tr).
__device__ __forceinline__ void v_frags_tr(const unsigned short* vb, bf16x8 a[4], int s,
                                           const int vl[4]) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const int kt = s >> 1, ks = s & 1;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    s4 r[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(vb + vl[dt] + (32 * kt + 8 * ks + 4 * h2) * 128));
    a[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

__device__ __forceinline__ void v_lane_offsets(int lane, int vl[4]) {
  asm volatile("" : "+v"(lane));
  const int s = lane & 15, grp = (lane >> 4) & 1, hf = lane >> 5;
  const int dsel = s & 3, k_lane = s >> 2;
  const int d_lane = ((dsel & 1) << 4) + ((dsel >> 1) << 2) + 8 * grp;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vl[dt] = (16 * hf + k_lane) * 128 + (4 * (dt ^ k_lane) + (d_lane >> 3)) * 8 + (d_lane & 7);
}

// Query rows of one tile's entries for one wave (rows 32w .. 32w + 31 = entries
// 32w/G .. (32w + 31)/G), held in vector registers until they are used. With
// G >= 4 a direct load of 4 rows stays within one entry, so every Q load address is a
// wave-uniform base plus a fixed lane offset; with G < 4 each lane holds its own row's query.
template <int G>
struct TileQ {
  static constexpr int EPW = G >= 4 ? 32 / G : 1;
  int q[EPW];

  // padding rows take the tile's last entry
  __device__ __forceinline__ void load(const int32_t* __restrict__ entry_q, const TileD& d,
                                       int wave, int rent) {
    const int last = d.e0 + max(d.n - 1, 0);
    int z = 0;
    asm volatile("" : "+v"(z));
    if constexpr (G >= 4) {
#pragma unroll
      for (int i = 0; i < EPW; ++i) q[i] = entry_q[min(d.e0 + wave * EPW + i, last) + z];
    } else {
      q[0] = entry_q[min(d.e0 + rent, last) + z];
    }
  }
  __device__ __forceinline__ int lane_query(int col) const {
    if constexpr (G >= 4) {
      int v = q[0];
#pragma unroll
      for (int i = 1; i < EPW; ++i) v = (col / G == i) ? q[i] : v;
      return v;
    } else {
      return q[0];
    }
  }
  // Q rows of the wave into its staging buffer (layout of dma_q); `qo` = lane offsets of
  // loads i % 4 (G >= 4).
  __device__ __forceinline__ void dma(u32x4* buf, const void* qp, int hq, int h, int g,
                                      const int qo[4], int lane) const {
    const char* const qb = reinterpret_cast<const char*>(qp);
    if constexpr (G >= 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row0 = __builtin_amdgcn_readfirstlane(q[(4 * i) / G]) * hq + h * G + (4 * i) % G;
        dma16s(qb + (size_t)row0 * 256, (uint32_t)qo[i & 3], lds_addr(buf + 64 * i));
      }
    } else {
      // rows of a load belong to several entries: per-lane addresses (dma_q's layout)
      const int rowidx = q[0] * hq + h * G + g;
      const int lr = lane / 16, lc = lane % 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int R = 4 * i + lr;
        const int src_row = __shfl(rowidx, R);
        dma16(qb + (size_t)src_row * 256 + (lc ^ (R % 16)) * 16, lds_addr(buf + 64 * i));
      }
    }
  }
};

// Lane offsets (bytes) of the Q row loads of TileQ::dma: load i brings rows 4i .. 4i + 3 of
// the wave, lane l taking chunk (l % 16) ^ ((4i + l / 16) % 16) of row 4i + l / 16.
__device__ __forceinline__ void q_lane_offsets(int lane, int qo[4]) {
  asm volatile("" : "+v"(lane));
  const int lr = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) qo[i] = lr * 256 + ((lc ^ (4 * i + lr)) * 16);
}

constexpr int kBufWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9)

// Buffer descriptor of `bytes` bytes at p, built from wave-uniform values (readfirstlane keeps
// the descriptor in scalar registers; a descriptor in vector registers would make the compiler
// wrap every access in a loop over its distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t srd(const void* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* const q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, 0, __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}

template <int G>
__global__ __launch_bounds__(512, 1) void attn_kv_tiled_kernel(KvTArgs a) {
  constexpr int MQ = 256 / G;          // entries per tile
  __shared__ u32x4 kvs[3][128 * 16];   // rotating K / V slots
  __shared__ u32x4 obuf_all[8][32 * 16];

  const int E = a.counters[0];
  if (E <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int r = wave * 32 + col;       // row of the tile
  const int rent = r / G, g = r % G;
  const int rp = rowperm(col), sw = swz(rp);
  u32x4* const obuf = obuf_all[wave];
  const int xcd = blockIdx.x % a.n_xcd, j = blockIdx.x / a.n_xcd;
  const float sl2 = a.scale_log2;
  const uint16_t* const kb = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* const vb = reinterpret_cast<const uint16_t*>(a.v);
  const uint32_t kv_row = (uint32_t)a.hkv * kD;
  int vl[4];
  v_lane_offsets(lane, vl);
  int ub[4];
  unstage_bases(lane, ub);
  int qo[4];
  q_lane_offsets(lane, qo);
  // byte offset of the lane's 16 bytes in read-back i < 4 (i >= 4: + 4 KiB)
  const int o_voff = (lane >> 4) * 256 + (lane & 15) * 16;

  // (sequence, group) of a phase
  auto seq_of = [&](int p, int* h) {
    *h = (p / a.n_r) % a.hkv;
    return load_seq_clamped(a.cu_q, a.cu_k, p / (a.n_r * a.hkv), a.total_q, a.total_k, a.max_q,
                            a.max_k);
  };
  auto kv_base = [&](const uint16_t* base, const Seq& sq, int h, int b) {
    return base + ((size_t)(sq.k0 + b * kBlock) * a.hkv + h) * kD;
  };

  TileIt it{xcd, 0, 0};
  it_enter(it, a, j);
  TileD d0 = it_decode(it_fetch(it, a, j), it, a, E);
  if (d0.n == 0) return;
  TileD d1 = it_decode(it_fetch(it, a, j), it, a, E);
  TileD d2 = it_decode(it_fetch(it, a, j), it, a, E);
  TileRaw r3 = it_fetch(it, a, j);

  int h0;
  Seq sq0 = seq_of(d0.p, &h0);
  int ks = 0, vs = 1, fs = 2;
  dma_block<false>(kvs[ks], kv_base(kb, sq0, h0, d0.b), kv_row, sq0.nk - d0.b * kBlock, wave, lane);
  dma_block<true>(kvs[vs], kv_base(vb, sq0, h0, d0.b), kv_row, sq0.nk - d0.b * kBlock, wave, lane);
  TileQ<G> tq0, tq1;
  tq0.load(a.entry_q, d0, wave, rent);
  wait_vm0();
  tq0.dma(obuf, a.q, a.hq, h0, g, qo, lane);
  bool opened = true;                  // the tile opens a bucket: K/V were just loaded

  bf16x8 bq[8];
  bf16x8 fr[2][4];
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float o_l = 0.f, o_lse = 0.f;
  // the previous tile's output rows: first partial row and row count (none yet)
  size_t o_row0 = 0;
  int o_nrow = 0;

  while (true) {
    const bool trans = d1.n != 0 && (d1.b != d0.b || d1.p != d0.p);
    int h1 = h0;
    Seq sq1 = sq0;
    if (d1.n != 0 && d1.p != d0.p) sq1 = seq_of(d1.p, &h1);
    const int u0 = d0.b * kBlock;
    const int nk_rel = sq0.nk - u0;
    int kmax = min(127, nk_rel - 1);
    if (a.causal) kmax = min(kmax, sq0.nk - sq0.nq + (tq0.lane_query(col) - sq0.q0) - u0);
    const bool need_mask = __any(kmax < 127);

    wait_vm0();               // Q rows (and, when `opened`, this bucket's K/V) have landed;
                              // tile records and entry queries read during the last tile too
    if (opened) __syncthreads();
    // reads for the coming tiles: entry queries of tile j + 1 (for its Q rows, loaded after
    // this tile's QK^T), the record of tile j + 4
    tq1 = tq0;
    if (d1.n) tq1.load(a.entry_q, d1, wave, rent);
    const TileD d3 = it_decode(r3, it, a, E);
    r3 = it_fetch(it, a, j);
    if (trans)
      dma_block<false>(kvs[fs], kv_base(kb, sq1, h1, d1.b), kv_row, sq1.nk - d1.b * kBlock, wave,
                       lane);
    read_q<false>(obuf, bq, col, hf);
    const u32x4* const kslot = kvs[ks];
    const unsigned short* const vslot = reinterpret_cast<const unsigned short*>(kvs[vs]);
    k_frags(*reinterpret_cast<const KVLds*>(kslot), fr[0], 0, rp, sw, hf);

    // ---- phase A: QK^T(j) | O(j-1) through LDS to memory: packed into LDS in steps 0-1,
    // read back one step ahead of its stores in steps 2-6; the staging buffer is then free
    // and the next tile's Q rows are requested in step 6
    f32x16 sc[4];
    u32x4 wb[2];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st < 7) k_frags(*reinterpret_cast<const KVLds*>(kslot), fr[(st + 1) & 1], st + 1, rp, sw, hf);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        sc[kt] = mfma32(fr[st & 1][kt], bq[st], st == 0 ? f32x16{} : sc[kt]);
      if (st < 2) {
        stage_o<false>(obuf, oacc[2 * st], 2 * st, 1.f, col, hf);
        stage_o<false>(obuf, oacc[2 * st + 1], 2 * st + 1, 1.f, col, hf);
      } else if (st < 7) {
        if (st > 2) {
          // streaming stores: the partials are read once, by the combine kernel
          const __amdgpu_buffer_rsrc_t ro = srd(a.part_o + o_row0 * kD, o_nrow * kD * 2);
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2)
            __builtin_amdgcn_raw_buffer_store_b128(wb[i2], ro, o_voff + (2 * (st - 3) + i2) * 1024, 0, 2);
        }
        if (st < 6) {
#pragma unroll
          for (int i2 = 0; i2 < 2; ++i2) {
            const int i = 2 * (st - 2) + i2;
            wb[i2] = obuf[ub[i & 3] + 256 * (i >> 2)];
          }
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                                srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                                srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 0);
          // Q of the next tile into the staging buffer, whose read-back is complete (the
          // stores above took its data from registers)
          tq1.dma(obuf, a.q, a.hq, h1, g, qo, lane);
        }
      }
      MSA_INTERLEAVE(1, 6);
    }
    if (trans) {
      __syncthreads();        // every wave is done with this bucket's K
      dma_block<true>(kvs[ks], kv_base(vb, sq1, h1, d1.b), kv_row, sq1.nk - d1.b * kBlock, wave,
                      lane);
    }
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
    v_frags_tr(vslot, fr[0], 0, vl);
    u32x4 pk[8];
    float l = exp_step(sc, 0, sl2, c, pk[0], 0.f);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st < 7) v_frags_tr(vslot, fr[(st + 1) & 1], st + 1, vl);
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
    o_nrow = max(0, min(32, d0.n * G - wave * 32));
    o_row0 = (size_t)d0.e0 * G + wave * 32;
    if (d1.n == 0) break;
    if (trans) {
      const int k2 = fs;
      fs = vs;
      vs = ks;
      ks = k2;
    }
    opened = trans;
    d0 = d1;
    d1 = d2;
    d2 = d3;
    sq0 = sq1;
    h0 = h1;
    tq0 = tq1;
  }
  // output of the last tile (after the last, unused, Q load into the buffer)
  wait_vm0();
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) stage_o<false>(obuf, oacc[dt], dt, 1.f, col, hf);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 w = obuf[ub[i & 3] + 256 * (i >> 2)];
    __builtin_amdgcn_raw_buffer_store_b128(w, srd(a.part_o + o_row0 * kD, o_nrow * kD * 2),
                                           o_voff + i * 1024, 0, 2);
  }
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                        srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                        srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 0);
}

template <int G>
hipError_t launch_kv_tiled_g(const KvTArgs& a, int n_wg, hipStream_t st) {
  hipLaunchKernelGGL((attn_kv_tiled_kernel<G>), dim3(n_wg), dim3(512), 0, st, a);
  return hipGetLastError();
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
  if (g.tiled) {
    KvTArgs t;
    t.q = q;
    t.k = k;
    t.v = v;
    t.scale_log2 = a.scale_log2;
    t.cu_q = cu_q;
    t.cu_k = cu_k;
    t.counters = a.counters;
    t.entry_q = a.entry_q;
    t.phase_base = reinterpret_cast<const int32_t*>(ws + L.phase_base);
    t.recs = reinterpret_cast<const int2*>(ws + L.tiles);
    t.part_lse = a.part_lse;
    t.part_l = a.part_l;
    t.part_o = a.part_o;
    t.total_q = s.total_q;
    t.total_k = s.total_k;
    t.max_q = s.max_q;
    t.max_k = s.max_k;
    t.hq = s.hq;
    t.hkv = s.hkv;
    t.nb_max = (int)g.nb_max;
    t.n_r = (int)g.n_r;
    t.n_phase = (int)g.n_phase;
    t.n_xcd = device_xcd_count();
    t.n_share = n_wg / t.n_xcd;
    t.causal = s.causal;
    switch (g.group) {
      case 1: return launch_kv_tiled_g<1>(t, n_wg, st);
      case 2: return launch_kv_tiled_g<2>(t, n_wg, st);
      case 4: return launch_kv_tiled_g<4>(t, n_wg, st);
      case 8: return launch_kv_tiled_g<8>(t, n_wg, st);
      default: return launch_kv_tiled_g<16>(t, n_wg, st);
    }
  }
  a.n_wg = n_wg;
  return s.dtype == MSA_FP8_E4M3 ? launch_kv_g<true>(a, g.group, n_wg, st)
                                 : launch_kv_g<false>(a, g.group, n_wg, st);
}

}  // namespace msa
