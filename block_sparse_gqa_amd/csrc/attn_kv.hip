// KV-outer (KV-stationary) main attention kernels.
//
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell" (summary and section 2): each
// selected KV block is loaded once and every query that chose it is gathered in; a work unit
// owns a single block, so there is one softmax step and no rescaling; partial outputs are
// written contiguously in work order. The GQA heads of one query form a contiguous box of Q
// rows, gathered with one index read per query-group.
//
// The plan cuts the entry order (sequence, group, query range, block, query) into tiles of
// 256 rows = 256/G entries of one bucket x G heads, 32 rows per wave, two waves per SIMD, and
// writes one record per tile. Each entry's G x D partial lands in rows e*G .. e*G+G-1 of the
// partial buffer, so a wave's 32 output rows are one contiguous range; they are written
// through a per-wave LDS buffer so that every store instruction covers 1 KiB of consecutive
// bytes. Two kernels walk the tiles: bf16 Q/K/V on bf16 MFMA, fp8 Q/K/V on fp8 MFMA.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {


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

// V^T operands (A) of key-step s (keys 32kt + 16hf + 8ks .. +7, kt = s/2, ks = s%2) for the
// 4 output-dim tiles, from a V^T block (row = head dim, 128 keys) in the layout of k_frags.
__device__ __forceinline__ void v_frags(const u32x4* vt, bf16x8 a[4], int s, int rp, int sw,
                                        int hf) {
  const int cc = (4 * (s >> 1) + 2 * hf + (s & 1)) ^ sw;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) a[dt] = as_bf16x8(vt[(dt * 32 + rp) * 16 + cc]);
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

// B operand of S^T from the staging buffer (chunk c of row R in slot c ^ (R % 16)):
// elements 16*st + 8*hf .. +7 of the lane's row.
__device__ __forceinline__ void read_q(const u32x4* buf, bf16x8 bq[8], int col, int hf) {
  asm volatile("" : "+v"(col), "+v"(hf));
  const int x = hf ^ (col & 15);          // (2st + hf) ^ (col % 16) == 2st ^ x
  const u32x4* const row = buf + col * 16;
#pragma unroll
  for (int st = 0; st < 8; ++st) bq[st] = as_bf16x8(row[(2 * st) ^ x]);
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

// ======================================================================================
// bf16: tiles of XCD-local query ranges, K/V restaged asynchronously.
//
// The plan cuts the entries of every (sequence, group, query range) phase into tiles of
// 256 / G entries of one bucket and writes one record per tile. Phase p belongs to XCD
// p % n_xcd (workgroup i runs on XCD i % n_xcd), whose n_share workgroups split the phase's
// tiles into contiguous shares; the Q rows of a phase (at most 4 MiB for 16 heads and 1024
// queries) stay in that XCD's L2 while every block of the range re-reads them.
//
// K and V blocks go to LDS by direct loads into three rotating 32 KiB slots. When the next
// tile starts a new bucket, its K block is loaded at the start of the current tile into the
// free slot (the V slot of the previous bucket, released by the barrier that opened the
// current bucket) and its V block, after a barrier, into the K slot of the current bucket once
// every wave has finished QK^T; the next tile starts after one more barrier. V comes from a
// transposed copy (transpose_v_kernel, one pass over V before the attention kernel), so its
// PV operands are plain 16-byte LDS reads like K's. Output stores go through buffer
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
  const float* descale;   // fp8: device [q, k, v] descales; bf16: unused
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
  const uint16_t* vw;     // bf16 V^T of each (group, key block) (fp8: widened exactly)
  int total_q, total_k, max_q, max_k;
  int hq, hkv, nb_max, n_r, n_phase, n_xcd, n_share, causal;
  int nbt;                // blocks per group of the transposed V (see transpose_v_kernel)
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

// A K block or a V^T block (128 rows of 256 bytes, the layout of k_frags and v_frags) into an
// LDS slot by the workgroup's 512 threads, 4 direct loads each: load p of wave w fills rows
// 32p + 4w .. +3, lane l fetching the chunk that belongs in its slot. Rows at or past nk_rel
// repeat the last one (K: keys past the sequence's end, whose scores are masked; a V^T block
// has all 128 rows).
__device__ __forceinline__ void dma_block(u32x4* dst, const uint16_t* base, uint32_t row_stride,
                                          int nk_rel, int wave, int lane) {
  const int slot = lane & 15;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 32 * p + 4 * wave + (lane >> 4);
    const int f = swz(row);
    const uint32_t r = (uint32_t)min(row, nk_rel - 1);
    dma16s(base, (r * row_stride + (uint32_t)((slot ^ f) * 8)) * 2,
           lds_addr(dst + p * 512 + wave * 64));
  }
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
  // Q rows of the wave into its staging buffer: load i brings rows 4i .. 4i + 3, lane l the
  // chunk that belongs in slot l % 16 of row 4i + l / 16 (chunk c of row R in slot
  // c ^ (R % 16)), 1 KiB of whole rows per load; `qo` = lane offsets of loads i % 4 (G >= 4).
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
      // rows of a load belong to several entries: per-lane addresses
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

// Lane offset that the buffer range check drops (a padding row, or no previous tile).
constexpr int kOffDrop = 0x40000000;

// Byte offset of the lane's row in the 8-row group layout of the partials, counted from the
// group of the wave's first row o_row0 (the store descriptor's base), plus the lane's half
// of a dim tile (chunks 4 dt + 2 hf + {0, 1}: 256 hf bytes); kOffDrop for rows past o_nrow.
__device__ __forceinline__ int store_lane_offset(size_t o_row0, int o_nrow, int col, int hf) {
  const int rr = (int)(o_row0 & 7) + col;
  return col < o_nrow ? ((rr >> 3) << 11) + ((rr & 7) << 4) + (hf << 8) : kOffDrop;
}

// Dim tile dt of a wave's output (lane (col, hf) holds dims 32 dt + 16 hf .. +15 of row col)
// from registers to the partial buffer: chunk 4 dt + 2 hf + j of each row, two stores that
// each cover 8 whole 128-byte lines when the rows fill their groups. Streaming stores: the
// partials are read once, by the combine kernel. The descriptor spans the (at most five)
// groups the wave's 32 rows touch; offsets past it (kOffDrop) are dropped by the hardware.
__device__ __forceinline__ void store_o_tile(char* part_o_b, size_t o_row0, const f32x16& o,
                                             int dt, int voff) {
  const __amdgpu_buffer_rsrc_t ro = srd(part_o_b + (o_row0 >> 3) * 2048, 5 * 2048);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[8 * j + 2 * i], o[8 * j + 2 * i + 1]);
    __builtin_amdgcn_raw_buffer_store_b128(w, ro, voff + (4 * dt + j) * 128, 0, 2);
  }
}

template <int G>
__global__ __launch_bounds__(512, 1) void attn_kv_tiled_kernel(KvTArgs a) {
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
  const uint32_t kv_row = (uint32_t)a.hkv * kD;
  int qo[4];
  q_lane_offsets(lane, qo);
  char* const part_o_b = reinterpret_cast<char*>(a.part_o);

  // (sequence, group) of a phase
  auto seq_of = [&](int p, int* h) {
    *h = (p / a.n_r) % a.hkv;
    return load_seq_clamped(a.cu_q, a.cu_k, p / (a.n_r * a.hkv), a.total_q, a.total_k, a.max_q,
                            a.max_k);
  };
  auto kv_base = [&](const uint16_t* base, const Seq& sq, int h, int b) {
    return base + ((size_t)(sq.k0 + b * kBlock) * a.hkv + h) * kD;
  };
  // V^T of block b of phase p's sequence, group h (blocks numbered as transpose_v_kernel does)
  auto vt_base = [&](int p, const Seq& sq, int h, int b) {
    const int s = p / (a.n_r * a.hkv);
    return a.vw + ((size_t)h * a.nbt + (size_t)(sq.k0 >> 7) + s + b) * (kD * kBlock);
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
  dma_block(kvs[ks], kv_base(kb, sq0, h0, d0.b), kv_row, sq0.nk - d0.b * kBlock, wave, lane);
  dma_block(kvs[vs], vt_base(d0.p, sq0, h0, d0.b), kBlock, kD, wave, lane);
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
  // the previous tile's output rows: first partial row, row count (none yet) and the lane's
  // byte offset in the 8-row group layout from the group of the first row
  size_t o_row0 = 0;
  int o_nrow = 0, o_voff = kOffDrop;

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
      dma_block(kvs[fs], kv_base(kb, sq1, h1, d1.b), kv_row, sq1.nk - d1.b * kBlock, wave,
                       lane);
    const u32x4* const kslot = kvs[ks];
    const u32x4* const vslot = kvs[vs];
    // A wave whose 32 rows all lie past the tile's entries (the last tile of a bucket) skips
    // the tile's math and Q rows: it only stores the previous tile's output and takes part in
    // the K/V loads and barriers.
    const bool act = d0.n * G > wave * 32;
    const bool act1 = d1.n * G > wave * 32;
    if (act) {
      f32x16 sc[4];
      read_q(obuf, bq, col, hf);
      k_frags(*reinterpret_cast<const KVLds*>(kslot), fr[0], 0, rp, sw, hf);
      // ---- phase A: QK^T(j) | O(j-1) from registers to memory in steps 0-3 (dim tile st:
      // two 16-byte chunks per lane, each store 8 whole 128-byte lines of the group layout);
      // the next tile's Q rows are requested in step 4, when this tile's Q operands have been
      // read (LDS reads complete in order, and the K operands of step 1 were read after them)
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st < 7) k_frags(*reinterpret_cast<const KVLds*>(kslot), fr[(st + 1) & 1], st + 1, rp, sw, hf);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sc[kt] = mfma32(fr[st & 1][kt], bq[st], st == 0 ? f32x16{} : sc[kt]);
        if (st < 4) {
          store_o_tile(part_o_b, o_row0, oacc[st], st, o_voff);
        } else if (st == 4) {
          // LSE and weight sum, streaming like the partials (both are read once, by the
          // combine): lines kept in L2 would only push out the phase's Q rows
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                                srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                                srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
          if (act1) tq1.dma(obuf, a.q, a.hq, h1, g, qo, lane);
        }
        MSA_INTERLEAVE(1, 6);
      }
      if (trans) {
        __syncthreads();        // every wave is done with this bucket's K
        dma_block(kvs[ks], vt_base(d1.p, sq1, h1, d1.b), kBlock, kD, wave, lane);
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
      v_frags(vslot, fr[0], 0, rp, sw, hf);
      u32x4 pk[8];
      float l = exp_step(sc, 0, sl2, c, pk[0], 0.f);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st < 7) v_frags(vslot, fr[(st + 1) & 1], st + 1, rp, sw, hf);
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
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) store_o_tile(part_o_b, o_row0, oacc[dt], dt, o_voff);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                            srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                            srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
      if (act1) tq1.dma(obuf, a.q, a.hq, h1, g, qo, lane);
      if (trans) {
        __syncthreads();
        dma_block(kvs[ks], vt_base(d1.p, sq1, h1, d1.b), kBlock, kD, wave, lane);
      }
    }
    o_nrow = max(0, min(32, d0.n * G - wave * 32));
    o_row0 = (size_t)d0.e0 * G + wave * 32;
    o_voff = store_lane_offset(o_row0, o_nrow, col, hf);
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
  for (int dt = 0; dt < 4; ++dt) store_o_tile(part_o_b, o_row0, oacc[dt], dt, o_voff);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                        srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                        srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
}

// ======================================================================================
// fp8: the tiled schedule with QK^T on the 8-bit MFMA (v_mfma_scale_f32_32x32x64_f8f6f4)
//
// Q and K stay OCP e4m3 in LDS (16 KiB per K block, 4 KiB of Q rows per wave), and each QK^T
// MFMA covers 64 of the contraction at twice the bf16 rate. For the 32x32x64 8-bit MFMA, lane l
// supplies row l % 32 of A (and column l % 32 of B) at contraction indices 32 (l / 32) .. +31,
// 32 bytes; the result has the 32x32 layout of the bf16 MFMA. QK^T: A = K rows (key order
// rowperm, as in the bf16 kernel), B = Q rows, D = 64 per MFMA (two MFMAs per 128 dims). The
// probabilities are rounded to bf16 and PV runs on bf16 MFMA, as in the bf16 kernel, against
// V widened to bf16 (exactly: every e4m3 value is a bf16 value) and transposed by the pass over
// V before the attention kernel; the V descale divides the stored weight sum instead of
// scaling V.
// Four 32 KiB slots (K in the first half of one): when the next tile opens a new bucket, its K
// and V blocks are both requested at the start of the current tile into the two slots the
// previous bucket left (released by the barrier that opened the current bucket), so a bucket
// change takes one barrier.

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c,
                                        int scale_a = 127) {
  // formats 0/0: e4m3 operands; scales are E8M0 codes (2^(code - 127)), B unscaled
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}

// LDS layouts (16-byte chunks, 8 per 128-byte row): chunk c of row r at slot c ^ f(r).
__device__ __forceinline__ int f8_swz_k(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
__device__ __forceinline__ int f8_swz_q(int r) { return (r ^ (r >> 3)) & 7; }

// An fp8 K block into an LDS slot by the workgroup's 512 threads, 2 direct loads each: load p
// of wave w fills rows 64p + 8w .. +7. Rows at or past nk_rel repeat the last key.
__device__ __forceinline__ void dma_block8(u32x4* dst, const uint8_t* base, uint32_t row_stride,
                                           int nk_rel, int wave, int lane) {
  const int slot = lane & 7;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = 64 * p + 8 * wave + (lane >> 3);
    const int f = f8_swz_k(row);
    const uint32_t r = (uint32_t)min(row, nk_rel - 1);
    dma16s(base, r * row_stride + (uint32_t)((slot ^ f) * 16), lds_addr(dst + p * 512 + wave * 64));
  }
}

// Entry queries of a wave's 32 rows (fp8: a 1 KiB load brings 8 rows, one entry when G >= 8).
template <int G>
struct TileQ8 {
  static constexpr int EPW = G >= 8 ? 32 / G : 1;
  int q[EPW];

  __device__ __forceinline__ void load(const int32_t* __restrict__ entry_q, const TileD& d,
                                       int wave, int rent) {
    const int last = d.e0 + max(d.n - 1, 0);
    int z = 0;
    asm volatile("" : "+v"(z));
    if constexpr (G >= 8) {
#pragma unroll
      for (int i = 0; i < EPW; ++i) q[i] = entry_q[min(d.e0 + wave * EPW + i, last) + z];
    } else {
      q[0] = entry_q[min(d.e0 + rent, last) + z];
    }
  }
  __device__ __forceinline__ int lane_query(int col) const {
    if constexpr (G >= 8) {
      int v = q[0];
#pragma unroll
      for (int i = 1; i < EPW; ++i) v = (col / G == i) ? q[i] : v;
      return v;
    } else {
      return q[0];
    }
  }
  // Q rows of the wave: load i brings rows 8i .. 8i + 7, lane l chunk (l % 8) ^ f8_swz_q(row)
  // of row 8i + l / 8 into slot l % 8 of that row.
  __device__ __forceinline__ void dma(u32x4* buf, const void* qp, int hq, int h, int g,
                                      int lane) const {
    const char* const qb = reinterpret_cast<const char*>(qp);
    const int lr = lane >> 3, lc = lane & 7;
    if constexpr (G >= 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row0 = __builtin_amdgcn_readfirstlane(q[(8 * i) / G]) * hq + h * G + (8 * i) % G;
        const int R = 8 * i + lr;
        dma16s(qb + (size_t)row0 * 128, (uint32_t)(lr * 128 + ((lc ^ f8_swz_q(R)) * 16)),
               lds_addr(buf + 64 * i));
      }
    } else {
      const int rowidx = q[0] * hq + h * G + g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int R = 8 * i + lr;
        const int src_row = __shfl(rowidx, R);
        dma16(qb + (size_t)src_row * 128 + (lc ^ f8_swz_q(R)) * 16, lds_addr(buf + 64 * i));
      }
    }
  }
};

// B operand of S^T for contraction step ds: Q[row col][64 ds + 32 hf .. +31].
__device__ __forceinline__ i32x8 read_q8(const u32x4* buf, int ds, int col, int hf) {
  const int f = f8_swz_q(col);
  const u32x4 lo = buf[col * 8 + ((4 * ds + 2 * hf) ^ f)];
  const u32x4 hi = buf[col * 8 + ((4 * ds + 2 * hf + 1) ^ f)];
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// A operand of S^T for key tile kt, contraction step ds: K[32 kt + rowperm(col)][64 ds + 32 hf ..].
__device__ __forceinline__ i32x8 read_k8(const u32x4* kb, int kt, int ds, int rp, int hf) {
  const int r = 32 * kt + rp;
  const int f = f8_swz_k(r);
  const u32x4 lo = kb[r * 8 + ((4 * ds + 2 * hf) ^ f)];
  const u32x4 hi = kb[r * 8 + ((4 * ds + 2 * hf + 1) ^ f)];
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
template <int G>
__global__ __launch_bounds__(512, 1) void attn_kv_f8_kernel(KvTArgs a) {
  __shared__ u32x4 kvs[4][128 * 16];   // fp8 K (first 16 KiB of a slot) and bf16 V slots
  __shared__ u32x4 obuf_all[8][32 * 8];

  const int E = a.counters[0];
  if (E <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int r = wave * 32 + col;       // row of the tile
  const int rent = r / G, g = r % G;
  const int rp = rowperm(col), vsw = swz(rp);
  u32x4* const obuf = obuf_all[wave];
  const int xcd = blockIdx.x % a.n_xcd, j = blockIdx.x / a.n_xcd;
  const float sl2 = a.scale_log2 * a.descale[0] * a.descale[1];
  // The partial output is accumulated against the raw e4m3 values of V (widened exactly to
  // bf16); its weight sum is stored divided by the V descale dv, so that output over weight
  // sum carries dv. dv = 0 gives an infinite weight sum: a zero contribution with the right
  // log-sum-exp.
  const float inv_dv = 1.f / a.descale[2];
  const uint8_t* const kb = reinterpret_cast<const uint8_t*>(a.k);
  const uint32_t k_row = (uint32_t)a.hkv * kD;     // bytes between consecutive fp8 keys
  char* const part_o_b = reinterpret_cast<char*>(a.part_o);

  auto seq_of = [&](int p, int* h) {
    *h = (p / a.n_r) % a.hkv;
    return load_seq_clamped(a.cu_q, a.cu_k, p / (a.n_r * a.hkv), a.total_q, a.total_k, a.max_q,
                            a.max_k);
  };
  auto k_base = [&](const Seq& sq, int h, int bb) {
    return kb + ((size_t)(sq.k0 + bb * kBlock) * a.hkv + h) * kD;
  };
  // V^T (widened) of block bb of phase p's sequence, group h (numbered as transpose_v_kernel does)
  auto vt_base = [&](int p, const Seq& sq, int h, int bb) {
    const int s = p / (a.n_r * a.hkv);
    return a.vw + ((size_t)h * a.nbt + (size_t)(sq.k0 >> 7) + s + bb) * (kD * kBlock);
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
  int ks_ = 0, vs_ = 1, fk_ = 2, fv_ = 3;
  dma_block8(kvs[ks_], k_base(sq0, h0, d0.b), k_row, sq0.nk - d0.b * kBlock, wave, lane);
  dma_block(kvs[vs_], vt_base(d0.p, sq0, h0, d0.b), kBlock, kD, wave, lane);
  TileQ8<G> tq0, tq1;
  tq0.load(a.entry_q, d0, wave, rent);
  wait_vm0();
  tq0.dma(obuf, a.q, a.hq, h0, g, lane);
  bool opened = true;

  bf16x8 fr[2][4];
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float o_l = 0.f, o_lse = 0.f;
  size_t o_row0 = 0;
  int o_nrow = 0, o_voff = kOffDrop;

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

    wait_vm0();               // Q rows (and, when `opened`, this bucket's K/V) have landed
    if (opened) __syncthreads();
    tq1 = tq0;
    if (d1.n) tq1.load(a.entry_q, d1, wave, rent);
    const TileD d3 = it_decode(r3, it, a, E);
    r3 = it_fetch(it, a, j);
    if (trans) {
      dma_block8(kvs[fk_], k_base(sq1, h1, d1.b), k_row, sq1.nk - d1.b * kBlock, wave, lane);
      dma_block(kvs[fv_], vt_base(d1.p, sq1, h1, d1.b), kBlock, kD, wave, lane);
    }
    const u32x4* const kslot = kvs[ks_];
    const u32x4* const vslot = kvs[vs_];
    // waves whose rows all lie past the tile's entries skip the tile's math and Q rows
    const bool act = d0.n * G > wave * 32;
    const bool act1 = d1.n * G > wave * 32;
    if (act) {
      const i32x8 bq0 = read_q8(obuf, 0, col, hf);
      const i32x8 bq1 = read_q8(obuf, 1, col, hf);

      // ---- phase A: QK^T(j) on the 8-bit MFMA (8 MFMAs) | O(j-1) from registers to memory,
      // dim tile kt after the MFMAs of key tile kt
      f32x16 sc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const i32x8 k0 = read_k8(kslot, kt, 0, rp, hf);
        const i32x8 k1 = read_k8(kslot, kt, 1, rp, hf);
        sc[kt] = mfma8(k0, bq0, f32x16{});
        sc[kt] = mfma8(k1, bq1, sc[kt]);
        store_o_tile(part_o_b, o_row0, oacc[kt], kt, o_voff);
      }
      // LSE and weight sum, streaming like the partials
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                            srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                            srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
      // Q of the next tile into the staging buffer: this tile's Q operands were read before the K
      // operands that the MFMAs above waited for (LDS reads complete in order)
      if (act1) tq1.dma(obuf, a.q, a.hq, h1, g, lane);
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
      // ---- phase B: PV(j) on bf16 MFMA against the widened V | exp of the next key-step
      v_frags(vslot, fr[0], 0, rp, vsw, hf);
      u32x4 pk[8];
      float l = exp_step(sc, 0, sl2, c, pk[0], 0.f);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st < 7) v_frags(vslot, fr[(st + 1) & 1], st + 1, rp, vsw, hf);
        const bf16x8 bp = as_bf16x8(pk[st]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          oacc[dt] = mfma32(fr[st & 1][dt], bp, st == 0 ? f32x16{} : oacc[dt]);
        if (st + 1 < 8) l = exp_step(sc, st + 1, sl2, c, pk[st + 1], l);
        MSA_INTERLEAVE(2, 7);
      }
      l += shfl_xor_f(l, 32);
      o_l = any ? l * inv_dv : 0.f;
      o_lse = any ? (c + log2f(l)) * 0.69314718055994531f : -__builtin_inff();
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) store_o_tile(part_o_b, o_row0, oacc[dt], dt, o_voff);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                            srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                            srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
      if (act1) tq1.dma(obuf, a.q, a.hq, h1, g, lane);
    }
    o_nrow = max(0, min(32, d0.n * G - wave * 32));
    o_row0 = (size_t)d0.e0 * G + wave * 32;
    o_voff = store_lane_offset(o_row0, o_nrow, col, hf);
    if (d1.n == 0) break;
    if (trans) {
      int x = ks_;
      ks_ = fk_;
      fk_ = x;
      x = vs_;
      vs_ = fv_;
      fv_ = x;
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
  for (int dt = 0; dt < 4; ++dt) store_o_tile(part_o_b, o_row0, oacc[dt], dt, o_voff);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_lse),
                                        srd(a.part_lse + o_row0, o_nrow * 4), col * 4, 0, 2);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o_l),
                                        srd(a.part_l + o_row0, o_nrow * 4), col * 4, 0, 2);
}

// V of every (sequence, group, key block) transposed for the PV operands, which are then read
// like K's (16 consecutive bytes per lane, no transpose loads); e4m3 V is widened to bf16 on
// the way (exactly: every e4m3 value is a bf16 value):
// vt[h][n][d][j] = V[k0 + 128 b + j][h][d] for block b of sequence s, n = k0 / 128 + s + b
// (k0 the sequence's first key: the blocks of different sequences are disjoint and
// n < ceil(total_k / 128) + batch), zero for keys past the sequence's end. One 128 x 128 tile
// per workgroup through LDS.
template <bool FP8>
__global__ __launch_bounds__(256) void transpose_v_kernel(const void* __restrict__ v,
                                                          uint16_t* __restrict__ vt,
                                                          const int32_t* cu_q, const int32_t* cu_k,
                                                          int total_q, int total_k, int max_q,
                                                          int max_k, int hkv, int nbt) {
  constexpr int TS = kD + 2;            // LDS row pitch (elements) of the [key][dim] tile
  __shared__ uint32_t t[kBlock * TS / 2];
  const int b = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  if (b * kBlock >= sq.nk) return;
  const int c = tid & 15;               // 8 dims 8c .. 8c + 7 of a key
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int key = 16 * p + (tid >> 4);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (b * kBlock + key < sq.nk) {
      const size_t e = ((size_t)(sq.k0 + b * kBlock + key) * hkv + h) * kD + 8 * c;
      if constexpr (FP8) {
        const u32x2 y = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(v) + e);
        const u32x2 lo = fp8x4_to_bf16x4(y[0]), hi = fp8x4_to_bf16x4(y[1]);
        x = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(v) + e);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) t[(key * TS + 8 * c) / 2 + i] = x[i];
  }
  __syncthreads();
  const uint16_t* th = reinterpret_cast<const uint16_t*>(t);
  uint16_t* out = vt + ((size_t)h * nbt + (size_t)(sq.k0 >> 7) + s + b) * (kD * kBlock);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int d = 16 * p + (tid >> 4);
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)th[(8 * c + 2 * i) * TS + d] | ((uint32_t)th[(8 * c + 2 * i + 1) * TS + d] << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + d * kBlock + 8 * c));
  }
}

template <int G>
hipError_t launch_kv_f8_g(const KvTArgs& a, int n_wg, hipStream_t st) {
  hipLaunchKernelGGL((attn_kv_f8_kernel<G>), dim3(n_wg), dim3(512), 0, st, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_kv_tiled_g(const KvTArgs& a, int n_wg, hipStream_t st) {
  hipLaunchKernelGGL((attn_kv_tiled_kernel<G>), dim3(n_wg), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_kv(const msa_shape& s, const Geometry& g, const Layout& L,
                          const void* q, const void* k, const void* v, const float* descale,
                          float scale, const int32_t* cu_q, const int32_t* cu_k, char* ws,
                          hipStream_t st) {
  if (g.n_words == 0) return hipSuccess;
  const int n_wg = device_cu_count();   // one workgroup (eight waves) per CU
  KvTArgs t;
  t.q = q;
  t.k = k;
  t.v = v;
  t.descale = descale;
  t.scale_log2 = scale * 1.4426950408889634f;
  t.cu_q = cu_q;
  t.cu_k = cu_k;
  t.counters = reinterpret_cast<const int32_t*>(ws + L.counters);
  t.entry_q = reinterpret_cast<const int32_t*>(ws + L.entry_q);
  t.phase_base = reinterpret_cast<const int32_t*>(ws + L.phase_base);
  t.recs = reinterpret_cast<const int2*>(ws + L.tiles);
  t.part_lse = reinterpret_cast<float*>(ws + L.part_lse);
  t.part_l = reinterpret_cast<float*>(ws + L.part_l);
  t.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o);
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
  t.vw = reinterpret_cast<const uint16_t*>(ws + L.v_wide);
  t.nbt = (int)(cdiv(s.total_k, kBlock) + s.batch);
  const dim3 tgrid((unsigned)g.nb_max, s.hkv, s.batch);
  uint16_t* const vt = reinterpret_cast<uint16_t*>(ws + L.v_wide);
  if (s.dtype == MSA_FP8_E4M3)
    hipLaunchKernelGGL(transpose_v_kernel<true>, tgrid, dim3(256), 0, st, v, vt, cu_q, cu_k,
                       s.total_q, s.total_k, s.max_q, s.max_k, s.hkv, t.nbt);
  else
    hipLaunchKernelGGL(transpose_v_kernel<false>, tgrid, dim3(256), 0, st, v, vt, cu_q, cu_k,
                       s.total_q, s.total_k, s.max_q, s.max_k, s.hkv, t.nbt);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.dtype == MSA_FP8_E4M3) {
    switch (g.group) {
      case 1: return launch_kv_f8_g<1>(t, n_wg, st);
      case 2: return launch_kv_f8_g<2>(t, n_wg, st);
      case 4: return launch_kv_f8_g<4>(t, n_wg, st);
      case 8: return launch_kv_f8_g<8>(t, n_wg, st);
      default: return launch_kv_f8_g<16>(t, n_wg, st);
    }
  }
  switch (g.group) {
    case 1: return launch_kv_tiled_g<1>(t, n_wg, st);
    case 2: return launch_kv_tiled_g<2>(t, n_wg, st);
    case 4: return launch_kv_tiled_g<4>(t, n_wg, st);
    case 8: return launch_kv_tiled_g<8>(t, n_wg, st);
    default: return launch_kv_tiled_g<16>(t, n_wg, st);
  }
}

}  // namespace msa
