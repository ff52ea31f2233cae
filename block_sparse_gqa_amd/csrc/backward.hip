// Main-branch backward over the selected blocks: dQ, dK, dV of exact softmax attention
// restricted to each query's union of selected keys ("Flash-MSA: accelerating million-token
// training": the block ids and the main branch's log-sum-exp are kept for the backward;
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell", section 2: KV-stationary work
// over the block -> query inverted index). With P = exp(tau S - LSE), D = rowsum(dO * O):
//   dV_b += P^T dO,  dP = dO V^T,  dS = P (dP - D),  dK_b += tau dS^T Q,  dQ += tau dS K_b.
//
// The inverted index of the forward's plan gives, for every (sequence, group, block), its
// entries (query rows) in each query range. bwd_kv_kernel: one workgroup of four waves per
// (sequence, group, block) stages K_b and V_b in LDS once and walks all its entries in tiles
// of 32 rows (32 / G entries x G heads); wave w owns keys 32 w .. 32 w + 31 and keeps their dK
// and dV in registers for the whole block, so every dK / dV row is written once, without
// atomics. Per tile, each wave forms S^T and dP^T for its keys on bf16 MFMA, P and dS in
// registers, then reads them back transposed through a small LDS buffer (16-bit transpose
// loads) for dV += P^T dO and dK += dS^T Q; the tile's dQ contribution of the wave's keys
// (dS K) is summed over the four waves in LDS and written, per entry, to a partial buffer that
// bwd_dq_kernel adds up per query (the entry order of the combine map).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));

// Transposed fragment of a row-major bf16 matrix in LDS (rs elements per row) for a 32x32x16
// MFMA operand: lane L gets column c0 + 16 ((L / 16) % 2) + L % 16 at rows r0 + 8 (L / 32) ..
// +7. ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j % 4 of the 8-byte
// pieces addressed by lanes 4 t + j / 4, t = 0..3; supplier lane i addresses row t' = i / 4,
// columns 4 (i % 4) .. +3, so lane j receives column (base + j) of rows t = 0..3.
__device__ __forceinline__ bf16x8 read_tr(const uint16_t* buf, int rs, int r0, int c0, int lane) {
  const int i = lane & 15, grp = (lane >> 4) & 1, kb = lane >> 5;
  const int col = c0 + 16 * grp + 4 * (i & 3);
  s4 r[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = r0 + 8 * kb + 4 * h2 + (i >> 2);
    r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(buf + row * rs + col));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct fragment (row-major, row = lane % 32, elements c0 + 8 (lane / 32) .. +7).
__device__ __forceinline__ bf16x8 read_rows(const uint16_t* buf, int rs, int r0, int c0,
                                            int lane) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + (r0 + (lane & 31)) * rs + c0 +
                                                   8 * (lane >> 5)));
}

// 128-wide bf16 tiles in LDS are stored with their 16-byte chunks XOR-swizzled by the row:
// chunk c of row r at c ^ f(r), f(r) = 4 (r % 4) + (r / 4) % 4, a permutation of 0..15 over
// 16 consecutive rows. A fragment read (32 rows, one chunk) then meets each of the 16 chunk
// positions twice, and a transpose load (4 consecutive rows x 4 consecutive chunks per half
// wave) all 16 once: r % 4 moves the chunk by whole groups of four.
__device__ __forceinline__ int sw(int row, int col) {
  const int f = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * kD + ((((col >> 3) ^ f) & 15) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x8 read_rows_sw(const uint16_t* buf, int r0, int c0, int lane) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + sw(r0 + (lane & 31),
                                                            c0 + 8 * (lane >> 5))));
}

__device__ __forceinline__ bf16x8 read_tr_sw(const uint16_t* buf, int r0, int c0, int lane) {
  const int i = lane & 15, grp = (lane >> 4) & 1, kb = lane >> 5;
  const int col = c0 + 16 * grp + 4 * (i & 3);
  s4 r[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = r0 + 8 * kb + 4 * h2 + (i >> 2);
    r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(buf + sw(row, col)));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// 32 x 32 bf16 tiles [row][key] (P and dS) with the 16-byte chunks of a row XOR-swizzled by
// row / 4, so that the row-per-lane writes and reads and the 4-row transpose loads, whose rows
// lie 64 bytes apart, spread over the banks.
__device__ __forceinline__ int pswz(int row, int key) {
  return row * 32 + ((((key >> 3) ^ (row >> 2)) & 3) << 3) + (key & 7);
}

// read_tr and read_rows over a pswz tile.
__device__ __forceinline__ bf16x8 read_tr_p(const uint16_t* buf, int r0, int c0, int lane) {
  const int i = lane & 15, grp = (lane >> 4) & 1, kb = lane >> 5;
  const int col = c0 + 16 * grp + 4 * (i & 3);
  s4 r[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = r0 + 8 * kb + 4 * h2 + (i >> 2);
    r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(buf + pswz(row, col)));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 read_rows_p(const uint16_t* buf, int c0, int lane) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + pswz(lane & 31, c0 + 8 * (lane >> 5))));
}

// Sum over aligned groups of N lanes (N <= 16, within a DPP row) as fused DPP adds: the moved
// operand is taken with a zero fill, which none of these in-row patterns ever uses, so the
// compiler folds each move into its add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_z(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (N >= 2) v += dpp_z<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_z<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_z<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_z<kDppMirror>(v);
  return v;
}

// D[t, h] = sum_d dO[t, h, d] O[t, h, d] (fp32): 16 lanes per row of 128, 16-byte loads.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       float* __restrict__ dsum, int rows) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
  if (row >= rows) return;
  const u32x4 x = *reinterpret_cast<const u32x4*>(o + (size_t)row * kD + 8 * c);
  const u32x4 y = *reinterpret_cast<const u32x4*>(dout + (size_t)row * kD + 8 * c);
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v += bf16_bits_to_f32(x[i] & 0xFFFFu) * bf16_bits_to_f32(y[i] & 0xFFFFu) +
         bf16_bits_to_f32(x[i] >> 16) * bf16_bits_to_f32(y[i] >> 16);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += shfl_xor_f(v, off);
  if (c == 0) dsum[row] = v;
}

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* dsum;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* offsets;
  const int32_t* entry_q;
  const int32_t* chunk_base;   // [n_cols + 1]: first chunk of each (sequence, group, block)
  const int32_t* col_of;       // [chunks]: the column of each chunk
  uint16_t* dq_part;           // [E][G][kD] bf16: each entry's dQ contribution
  float* dkv_part;             // [chunks][2][kBlock][kD]: dK, dV of chunks of split columns
  float* dk;
  float* dv;
  float scale, scale_log2;
  int total_q, total_k, max_q, max_k, hq, hkv, nb_max, wr, n_r, causal, chunk_e;
};

// Entries of column (s, g, b) over all query ranges: bucket (s, g, r, b) holds
// offsets[bk wr] .. offsets[(bk + 1) wr].
__device__ __forceinline__ size_t bucket_at(const BwdArgs& a, int s, int g, int r, int b) {
  return (((size_t)s * a.hkv + g) * a.n_r + r) * a.nb_max + b;
}

// Walk over the tiles of one chunk: the chunk's entries [lo, hi) of the column, numbered
// across the query ranges in order, cut per range segment into tiles of TE entries.
struct TileIt {
  int r, base, et, e1;
};

__device__ __forceinline__ bool next_segment(const BwdArgs& a, int s, int g, int b, int lo,
                                             int hi, TileIt& it) {
  while (it.r < a.n_r && it.base < hi) {
    const size_t bk = bucket_at(a, s, g, it.r, b);
    const int f0 = a.offsets[bk * a.wr], f1 = a.offsets[(bk + 1) * a.wr];
    const int e0 = f0 + max(lo - it.base, 0), e1 = f0 + min(hi - it.base, f1 - f0);
    it.base += f1 - f0;
    ++it.r;
    if (e0 < e1) {
      it.et = e0;
      it.e1 = e1;
      return true;
    }
  }
  return false;
}

template <int G>
__global__ __launch_bounds__(512, 1) void bwd_kv_kernel(BwdArgs a) {
  constexpr int TE = 64 / G;                 // entries per tile of 64 rows
  __shared__ uint16_t kb[kBlock * kD];       // K_b, V_b (swizzled)
  __shared__ uint16_t vb[kBlock * kD];
  __shared__ uint16_t qt[2][64 * kD];        // the tile's Q and dO rows, double-buffered
  __shared__ uint16_t dot[2][64 * kD];
  __shared__ uint16_t pbuf[8][32 * 32];      // per wave: P and dS of its keys and rows,
  __shared__ uint16_t sbuf[8][32 * 32];      //   [row][key]

  const int chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave w: keys 32 kw .. +31 of the block; rows 32 hw .. +31 of the tile for S, dP and dQ;
  // dims 64 hw .. +63 of dK and dV (the two waves of a key quarter split the dims)
  const int kw = wave & 3, hw = wave >> 2;
  const int col = lane & 31, hf = lane >> 5;
  const int cl = a.col_of[chunk];            // -1: past the last chunk
  if (cl < 0) return;
  const int b = cl % a.nb_max, g = (cl / a.nb_max) % a.hkv, s = cl / (a.nb_max * a.hkv);
  const int j = chunk - a.chunk_base[cl];
  const bool split = a.chunk_base[cl + 1] - a.chunk_base[cl] > 1;
  const int lo = j * a.chunk_e, hi = lo + a.chunk_e;   // the chunk's entries of the column
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int u0 = b * kBlock;

  // K_b and V_b (rows past the sequence repeat its last key; their weights are masked)
  for (int i = tid; i < kBlock * kD / 8; i += 512) {
    const int row = i / (kD / 8), c = i % (kD / 8);
    const size_t src = ((size_t)(sq.k0 + min(u0 + row, sq.nk - 1)) * a.hkv + g) * kD + 8 * c;
    *reinterpret_cast<u32x4*>(kb + sw(row, 8 * c)) = *reinterpret_cast<const u32x4*>(a.k + src);
    *reinterpret_cast<u32x4*>(vb + sw(row, 8 * c)) = *reinterpret_cast<const u32x4*>(a.v + src);
  }

  f32x16 dk_acc[2], dv_acc[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }
  const int key0 = 32 * kw;                  // this wave's keys within the block
  const int row0 = 32 * hw;                  // this wave's rows within the tile

  // Staging rows of this thread: n = tid / 16 + 32 k (k = 0, 1), 16-byte column tid % 16.
  // Compute row of this lane: n = row0 + col. Loads of a tile: entry rows first, then Q, dO,
  // LSE, D.
  const int c16 = tid % 16;
  auto load_rows = [&](int et, int e1, int eq[2], int& eqc) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = et + (tid / 16 + 32 * k) / G;
      eq[k] = e < e1 ? a.entry_q[e] : -1;
    }
    const int e = et + (row0 + col) / G;
    eqc = e < e1 ? a.entry_q[e] : -1;
  };
  auto load_data = [&](const int eq[2], int eqc, u32x4 qv[2], u32x4 ov[2], float& lse2,
                       float& dsum) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int n = tid / 16 + 32 * k;
      qv[k] = u32x4{0u, 0u, 0u, 0u};
      ov[k] = u32x4{0u, 0u, 0u, 0u};
      if (eq[k] >= 0) {
        const size_t row = (size_t)eq[k] * a.hq + g * G + n % G;
        qv[k] = *reinterpret_cast<const u32x4*>(a.q + row * kD + 8 * c16);
        ov[k] = *reinterpret_cast<const u32x4*>(a.dout + row * kD + 8 * c16);
      }
    }
    lse2 = 0.f;
    dsum = 0.f;
    if (eqc >= 0) {
      const size_t hrow = (size_t)eqc * a.hq + g * G + (row0 + col) % G;
      lse2 = a.lse[hrow] * 1.4426950408889634f;
      dsum = a.dsum[hrow];
    }
  };
  auto store_slot = [&](int slot, const u32x4 qv[2], const u32x4 ov[2]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int n = tid / 16 + 32 * k;
      *reinterpret_cast<u32x4*>(qt[slot] + sw(n, 8 * c16)) = qv[k];
      *reinterpret_cast<u32x4*>(dot[slot] + sw(n, 8 * c16)) = ov[k];
    }
  };

  __syncthreads();                           // K_b, V_b staged
  // the wave's K rows as A operands of S^T, kept for the whole chunk (V's are read from LDS)
  bf16x8 kf[kD / 16];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) kf[ks] = read_rows_sw(kb, key0, 16 * ks, lane);

  TileIt it{0, 0, 0, 0};
  bool have = next_segment(a, s, g, b, lo, hi, it);
  int cur_et = it.et, cur_e1 = it.e1;
  int eq[2] = {-1, -1}, eqc = -1;
  u32x4 qv[2], ov[2];
  float lse2 = 0.f, dsum = 0.f;
  if (have) {
    load_rows(cur_et, cur_e1, eq, eqc);
    load_data(eq, eqc, qv, ov, lse2, dsum);
    store_slot(0, qv, ov);
  }
  int cur_t = eqc;
  // the following tile
  it.et += TE;
  bool have_next = have && (it.et < it.e1 || next_segment(a, s, g, b, lo, hi, it));
  int slot = 0;

  while (have) {
    __syncthreads();                         // slot written; last tile's P / dS reads done
    const int nx_et = it.et, nx_e1 = it.e1;
    int nq[2] = {-1, -1}, nqc = -1;
    if (have_next) load_rows(nx_et, nx_e1, nq, nqc);

    const bool row_ok = cur_t >= 0;
    const int pos = sq.nk - sq.nq + (cur_t - sq.q0);
    const uint16_t* const qs = qt[slot];
    const uint16_t* const os = dot[slot];
    // S^T and dP^T for the wave's 32 keys x its 32 rows of the tile
    f32x16 st = {}, dpt = {};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const bf16x8 qb = read_rows_sw(qs, row0, 16 * ks, lane);
      const bf16x8 ob = read_rows_sw(os, row0, 16 * ks, lane);
      st = mfma32(kf[ks], qb, st);
      dpt = mfma32(read_rows_sw(vb, key0, 16 * ks, lane), ob, dpt);
    }
    // P = exp(tau S - LSE) on visible keys; dS = P (dP - D); both to the wave's buffers as
    // [row][key] (lane (row col, half hf) holds keys 8 (r / 4) + 4 hf + r % 4 in st[r])
    uint16_t* const pb = pbuf[wave];
    uint16_t* const sb = sbuf[wave];
    // the row's visible keys among the wave's: key0 + m with m <= kmax
    int kmax = min(kBlock - 1, sq.nk - 1 - u0) - key0;
    if (a.causal) kmax = min(kmax, pos - u0 - key0);
    if (!(row_ok && lse2 > -__builtin_inff())) kmax = -1;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float p[4], d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = 8 * q4 + 4 * hf + i <= kmax;
        p[i] = vis ? __builtin_amdgcn_exp2f(fmaf(st[4 * q4 + i], a.scale_log2, -lse2)) : 0.f;
        d[i] = p[i] * (dpt[4 * q4 + i] - dsum);
      }
      u32x2 pw, sw2;
      pw[0] = pack_bf16x2(p[0], p[1]);
      pw[1] = pack_bf16x2(p[2], p[3]);
      sw2[0] = pack_bf16x2(d[0], d[1]);
      sw2[1] = pack_bf16x2(d[2], d[3]);
      *reinterpret_cast<u32x2*>(pb + pswz(col, 8 * q4 + 4 * hf)) = pw;
      *reinterpret_cast<u32x2*>(sb + pswz(col, 8 * q4 + 4 * hf)) = sw2;
    }
    // the following tile's data, in flight during the products below
    if (have_next) load_data(nq, nqc, qv, ov, lse2, dsum);
    __syncthreads();                         // P, dS of every wave written

    // dQ of the wave's 32 rows, dims 32 kw .. +31, over all 128 keys: dS[rows][keys] K[keys][dims]
    // (before dK / dV, so that its partial stores drain under the dK / dV products)
    f32x16 dq = {};
#pragma unroll
    for (int kk = 0; kk < kBlock / 16; ++kk) {
      const bf16x8 s0 = read_rows_p(sbuf[(kk >> 1) + 4 * hw], 16 * (kk & 1), lane);
      const bf16x8 k0 = read_tr_sw(kb, 16 * kk, 32 * kw, lane);
      dq = mfma32(s0, k0, dq);
    }
    // stores: the lanes of dims 2c and 2c + 1 swap one value per pair of rows (DPP), so that
    // each writes two adjacent dims of one row as a 4-byte piece (half the store instructions)
    const bool odd = col & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float lo = dq[2 * i] * a.scale, hi = dq[2 * i + 1] * a.scale;
      const float got = __int_as_float(
          __builtin_amdgcn_mov_dpp(__float_as_int(odd ? lo : hi), 0xB1, 0xF, 0xF, false));
      const int rr = 2 * i + (odd ? 1 : 0);
      const int n = row0 + 8 * (rr / 4) + 4 * hf + rr % 4;
      const int e = cur_et + n / G;
      // streaming stores: each partial is read once, by bwd_dq_kernel; lines kept in L2 would
      // only push out the tiles' Q and dO rows
      if (e < cur_e1)
        __builtin_nontemporal_store(
            odd ? pack_bf16x2(got, hi) : pack_bf16x2(lo, got),
            reinterpret_cast<uint32_t*>(a.dq_part + ((size_t)e * G + n % G) * kD + 32 * kw + (col & ~1)));
    }
    // dV += P^T dO, dK += dS^T Q for the wave's keys and dims 64 hw .. +63: contraction over
    // the tile's 64 rows (rows 0-31 in the buffers of waves kw, rows 32-63 in those of kw + 4)
#pragma unroll
    for (int kr = 0; kr < 4; ++kr) {
      const int src = kw + 4 * (kr >> 1);
      const bf16x8 pa = read_tr_p(pbuf[src], 16 * (kr & 1), 0, lane);   // P^T[key][rows]
      const bf16x8 sa = read_tr_p(sbuf[src], 16 * (kr & 1), 0, lane);   // dS^T[key][rows]
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 ob = read_tr_sw(os, 16 * kr, 64 * hw + 32 * dt, lane);   // dO[rows][dims]
        const bf16x8 qb = read_tr_sw(qs, 16 * kr, 64 * hw + 32 * dt, lane);   // Q[rows][dims]
        dv_acc[dt] = mfma32(pa, ob, dv_acc[dt]);
        dk_acc[dt] = mfma32(sa, qb, dk_acc[dt]);
      }
    }
    if (have_next) store_slot(slot ^ 1, qv, ov);
    slot ^= 1;
    have = have_next;
    cur_et = nx_et;
    cur_e1 = nx_e1;
    cur_t = nqc;
    if (have) {
      it.et += TE;
      have_next = it.et < it.e1 || next_segment(a, s, g, b, lo, hi, it);
    }
  }
  if (split) {                              // partials, summed per column in chunk order
    float* const pk = a.dkv_part + (size_t)chunk * 2 * kBlock * kD;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int m = key0 + 8 * (rr / 4) + 4 * hf + rr % 4;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        __builtin_nontemporal_store(dk_acc[dt][rr] * a.scale, pk + m * kD + 64 * hw + 32 * dt + col);
        __builtin_nontemporal_store(dv_acc[dt][rr], pk + (kBlock + m) * kD + 64 * hw + 32 * dt + col);
      }
    }
    return;
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int u = u0 + key0 + 8 * (rr / 4) + 4 * hf + rr % 4;
    if (u < sq.nk) {
      const size_t row = ((size_t)(sq.k0 + u) * a.hkv + g) * kD + 64 * hw;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        a.dk[row + 32 * dt + col] = dk_acc[dt][rr] * a.scale;
        a.dv[row + 32 * dt + col] = dv_acc[dt][rr];
      }
    }
  }
}

// Chunks of every column (s, g, b): ceil(entries / chunk_e), at least one for a block that
// lies in its sequence (its dK, dV rows are written even when no query chose it), none past
// it. One workgroup scans the columns in order: chunk_base, the chunk -> column map, and -1
// for the unused tail of the map (the grid is sized for the bound).
__global__ __launch_bounds__(256) void bwd_chunks_kernel(BwdArgs a, int32_t* chunk_base,
                                                         int32_t* col_of, int n_cols,
                                                         int chunks_max) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int run = 0;
  for (int c0 = 0; c0 < n_cols; c0 += 256) {
    const int c = c0 + tid;
    int n = 0;
    if (c < n_cols) {
      const int b = c % a.nb_max, g = (c / a.nb_max) % a.hkv, s = c / (a.nb_max * a.hkv);
      const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q,
                                      a.max_k);
      if (b * kBlock < sq.nk) {
        int e = 0;
        for (int r = 0; r < a.n_r; ++r) {
          const size_t bk = bucket_at(a, s, g, r, b);
          e += a.offsets[(bk + 1) * a.wr] - a.offsets[bk * a.wr];
        }
        n = max(1, (e + a.chunk_e - 1) / a.chunk_e);
      }
    }
    int x = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int pre = run, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pre += (w < wave) ? wsum[w] : 0;
      tot += wsum[w];
    }
    __syncthreads();
    pre += x - n;
    if (c < n_cols) {
      chunk_base[c] = pre;
      for (int i = 0; i < n && pre + i < chunks_max; ++i) col_of[pre + i] = c;
    }
    run += tot;
  }
  if (tid == 0) chunk_base[n_cols] = run;
  for (int i = run + tid; i < chunks_max; i += 256) col_of[i] = -1;
}

// dK, dV of split columns: the chunks' partials added in chunk order (deterministic). Eight
// workgroups per column, each over 1 / 8 of its 2 x 128 x 128 values.
constexpr int kReduceParts = 8;
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(BwdArgs a) {
  const int cl = blockIdx.x, tid = threadIdx.x;
  constexpr int kPer = 2 * kBlock * kD / 4 / kReduceParts;   // float4 values per workgroup
  const int c0 = a.chunk_base[cl], c1 = a.chunk_base[cl + 1];
  if (c1 - c0 < 2) return;
  const int b = cl % a.nb_max, g = (cl / a.nb_max) % a.hkv, s = cl / (a.nb_max * a.hkv);
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  for (int i = (int)blockIdx.y * kPer + tid; i < ((int)blockIdx.y + 1) * kPer; i += 256) {
    const int m = (i / (kD / 4)) % kBlock, which = i / (kBlock * kD / 4);
    const int u = b * kBlock + m;
    if (u >= sq.nk) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = c0; c < c1; ++c)
      acc += reinterpret_cast<const f32x4*>(a.dkv_part + (size_t)c * 2 * kBlock * kD)[i];
    float* const dst = which ? a.dv : a.dk;
    reinterpret_cast<f32x4*>(dst + ((size_t)(sq.k0 + u) * a.hkv + g) * kD)[i % (kD / 4)] = acc;
  }
}

// dQ[t, h] = sum over the (query, group)'s entries of their partials (the combine map), in slot
// order. A thread owns 8 dims (16 bytes of a partial row) of one head; the partial loads of
// every slot are issued before any is added, each wave reading whole 256-byte head rows.
__global__ __launch_bounds__(256) void bwd_dq_kernel(const int32_t* __restrict__ cmap,
                                                     const uint16_t* __restrict__ dq_part,
                                                     float* __restrict__ dq, int64_t n, int hq,
                                                     int group, int topk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % 16);
  const int64_t row = i / 16;                // query row * hq + head
  const int head = (int)(row % hq), h = head / group, gi = head % group;
  const int64_t t = row / hq;
  const int32_t* cm = cmap + (t * (hq / group) + h) * topk;
  int es[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) es[k] = k < topk ? cm[k] : -1;
  u32x4 w[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    w[k] = u32x4{0u, 0u, 0u, 0u};
    if (es[k] >= 0)
      w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          dq_part + ((size_t)es[k] * group + gi) * kD + 8 * c));
  }
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    a0[0] += bf16_bits_to_f32(w[k][0] & 0xFFFFu);
    a0[1] += bf16_bits_to_f32(w[k][0] >> 16);
    a0[2] += bf16_bits_to_f32(w[k][1] & 0xFFFFu);
    a0[3] += bf16_bits_to_f32(w[k][1] >> 16);
    a1[0] += bf16_bits_to_f32(w[k][2] & 0xFFFFu);
    a1[1] += bf16_bits_to_f32(w[k][2] >> 16);
    a1[2] += bf16_bits_to_f32(w[k][3] & 0xFFFFu);
    a1[3] += bf16_bits_to_f32(w[k][3] >> 16);
  }
  f32x4* const out = reinterpret_cast<f32x4*>(dq + row * kD + 8 * c);
  out[0] = a0;
  out[1] = a1;
}

// The combine map of rows that lie in no sequence is never written by the plan: clear it.
__global__ __launch_bounds__(256) void bwd_clear_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = -1;
}

// ---------------------------------------------------------------------------------------
// Proxy (index-branch) backward. Per (query, group) over the same selected keys as the main
// branch: T = the main weights averaged over the group's G heads (recomputed from Q, K and
// the main LSE; held fixed), Pp = exp(tau_p z - LSEp) with z = q_idx . k_idx, and the
// gradients of sum KL(T || Pp): dz = tau_p (Pp - T), dq_idx = dz k_idx, dk_idx = dz^T q_idx.
// The proxy LSE is recomputed over the sparse keys first, block by block over the plan.

struct ProxyArgs {
  BwdArgs b;                   // main-branch fields: Q, K, main LSE, plan, chunks
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const float* lsep;           // [total_q, hkv] proxy LSE (natural log)
  float* dqi_part;             // [E][dp]: each entry's dq_idx contribution
  float* dki_part;             // [chunks][kBlock][dp]: dk_idx of chunks of split columns
  float* dk_idx;
  float pscale, pscale_log2;
};

// Proxy LSE in the KV-stationary order of the plan: per chunk of a (sequence, group, block)
// column, each wave holds the block's proxy keys as MFMA operands (key 32 kt + lane % 32, dims
// 16 ks + 8 (lane / 32) .. +7) and reduces the proxy scores of 32 entries at a time over the
// block's visible keys to a (max, sum) pair per entry, in log2 units: the block's proxy keys
// are read once per chunk, not once per query that selected the block. The pairs of a
// (query, group) are merged by proxy_lse_merge_kernel through the combine map.
template <int DP>
__global__ __launch_bounds__(256) void proxy_lse_part_kernel(ProxyArgs pa, float* __restrict__ pm,
                                                             float* __restrict__ pl) {
  const BwdArgs& a = pa.b;
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int cl = a.col_of[chunk];
  if (cl < 0) return;
  const int b = cl % a.nb_max, g = (cl / a.nb_max) % a.hkv, s = cl / (a.nb_max * a.hkv);
  const int j = chunk - a.chunk_base[cl];
  const int lo = j * a.chunk_e, hi = lo + a.chunk_e;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int u0 = b * kBlock;
  bf16x8 kf[4][DP / 16];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int u = min(u0 + 32 * kt + col, sq.nk - 1);
    const uint16_t* kr = pa.k_idx + ((size_t)(sq.k0 + u) * a.hkv + g) * DP + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks)
      kf[kt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 16 * ks));
  }
  TileIt it{0, 0, 0, 0};
  while (next_segment(a, s, g, b, lo, hi, it)) {
    for (int et = it.et + 32 * wave; et < it.e1; et += 128) {
      const int e = et + col;
      const int t = e < it.e1 ? a.entry_q[e] : -1;
      bf16x8 qf[DP / 16];
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (t >= 0)
          w = *reinterpret_cast<const u32x4*>(pa.q_idx + ((size_t)t * a.hkv + g) * DP + 16 * ks +
                                              8 * hf);
        qf[ks] = as_bf16x8(w);
      }
      f32x16 z[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        z[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < DP / 16; ++ks) z[kt] = mfma32(kf[kt][ks], qf[ks], z[kt]);
      }
      // visible keys of the entry: in the sequence and, causal, not after its query
      const int pos = sq.nk - sq.nq + (t - sq.q0);
      int kmax = min(kBlock - 1, sq.nk - 1 - u0);
      if (a.causal) kmax = min(kmax, pos - u0);
      if (t < 0) kmax = -1;
      float m = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = 32 * kt + 8 * (rr >> 2) + 4 * hf + (rr & 3);
          if (key <= kmax) m = fmaxf(m, z[kt][rr] * pa.pscale_log2);
        }
      m = fmaxf(m, shfl_xor_f(m, 32));
      float l = 0.f;
      if (m > -__builtin_inff()) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int key = 32 * kt + 8 * (rr >> 2) + 4 * hf + (rr & 3);
            if (key <= kmax) l += __builtin_amdgcn_exp2f(fmaf(z[kt][rr], pa.pscale_log2, -m));
          }
      }
      l += shfl_xor_f(l, 32);
      if (hf == 0 && t >= 0) {
        pm[e] = m;
        pl[e] = l;
      }
    }
  }
}

// Proxy LSE of each (query, group) (natural log): its entries' (max, sum) pairs merged in slot
// order through the combine map; -inf when no selected key is visible.
__global__ __launch_bounds__(256) void proxy_lse_merge_kernel(const int32_t* __restrict__ cmap,
                                                              const int32_t* __restrict__ counters,
                                                              const float* __restrict__ pm,
                                                              const float* __restrict__ pl,
                                                              float* __restrict__ lsep, int64_t n,
                                                              int topk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int n_ent = counters[0];
  const int32_t* cm = cmap + i * topk;
  float m = -__builtin_inff();
  for (int k = 0; k < topk; ++k) {
    const int e = cm[k];
    if (e >= 0 && e < n_ent) m = fmaxf(m, pm[e]);
  }
  float l = 0.f;
  if (m > -__builtin_inff())
    for (int k = 0; k < topk; ++k) {
      const int e = cm[k];
      if (e >= 0 && e < n_ent && pm[e] > -__builtin_inff())
        l += pl[e] * __builtin_amdgcn_exp2f(pm[e] - m);
    }
  lsep[i] = m > -__builtin_inff() ? (m + log2f(l)) * 0.6931471805599453f : -__builtin_inff();
}

template <int G, int DP>
__global__ __launch_bounds__(256, 1) void proxy_bwd_kernel(ProxyArgs pa) {
  const BwdArgs& a = pa.b;
  constexpr int TE = 32 / G;
  __shared__ uint16_t kb[kBlock * kD];       // K_b (swizzled)
  __shared__ uint16_t kib[kBlock * DP];      // k_idx of the block, row-major
  __shared__ uint16_t qt[2][32 * kD];        // the tile's Q rows (swizzled), double-buffered
  __shared__ uint16_t qit[2][32 * DP];       // row n: q_idx of the entry of row n
  __shared__ uint16_t zbuf[4][32 * 32];      // per wave: dz / G of its keys, [row][key]

  const int chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int cl = a.col_of[chunk];
  if (cl < 0) return;
  const int b = cl % a.nb_max, g = (cl / a.nb_max) % a.hkv, s = cl / (a.nb_max * a.hkv);
  const int j = chunk - a.chunk_base[cl];
  const bool split = a.chunk_base[cl + 1] - a.chunk_base[cl] > 1;
  const int lo = j * a.chunk_e, hi = lo + a.chunk_e;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int u0 = b * kBlock;

  for (int i = tid; i < kBlock * kD / 8; i += 256) {
    const int row = i / (kD / 8), c = i % (kD / 8);
    const size_t src = ((size_t)(sq.k0 + min(u0 + row, sq.nk - 1)) * a.hkv + g) * kD + 8 * c;
    *reinterpret_cast<u32x4*>(kb + sw(row, 8 * c)) = *reinterpret_cast<const u32x4*>(a.k + src);
  }
  for (int i = tid; i < kBlock * DP / 8; i += 256) {
    const int row = i / (DP / 8), c = i % (DP / 8);
    const size_t src = ((size_t)(sq.k0 + min(u0 + row, sq.nk - 1)) * a.hkv + g) * DP + 8 * c;
    *reinterpret_cast<u32x4*>(kib + row * DP + 8 * c) =
        *reinterpret_cast<const u32x4*>(pa.k_idx + src);
  }
  __syncthreads();
  const int key0 = 32 * wave;
  bf16x8 kf[kD / 16], kif[DP / 16];
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) kf[ks] = read_rows_sw(kb, key0, 16 * ks, lane);
#pragma unroll
  for (int ks = 0; ks < DP / 16; ++ks) kif[ks] = read_rows(kib, DP, key0, 16 * ks, lane);
  f32x16 acc[DP / 32];
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) acc[dt] = f32x16{};

  // a tile's loads: entry rows (Q staging rows tid / 16 + 16 k, proxy row tid / (DP / 8), the
  // lane's compute row col), then Q, q_idx, the main LSE and the proxy LSE
  auto load_rows = [&](int et, int e1, int eq[2], int& eqi, int& eqc) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = et + (tid / 16 + 16 * k) / G;
      eq[k] = e < e1 ? a.entry_q[e] : -1;
    }
    const int ei = et + (tid / (DP / 8)) / G;
    eqi = (tid < 4 * DP && ei < e1) ? a.entry_q[ei] : -1;
    const int e = et + col / G;
    eqc = e < e1 ? a.entry_q[e] : -1;
  };
  auto load_data = [&](const int eq[2], int eqi, int eqc, u32x4 qv[2], u32x4& pv, float& lse2,
                       float& lsep2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int n = tid / 16 + 16 * k;
      qv[k] = u32x4{0u, 0u, 0u, 0u};
      if (eq[k] >= 0)
        qv[k] = *reinterpret_cast<const u32x4*>(
            a.q + ((size_t)eq[k] * a.hq + g * G + n % G) * kD + 8 * (tid % 16));
    }
    pv = u32x4{0u, 0u, 0u, 0u};
    if (eqi >= 0)
      pv = *reinterpret_cast<const u32x4*>(pa.q_idx + ((size_t)eqi * a.hkv + g) * DP +
                                           8 * (tid % (DP / 8)));
    lse2 = -__builtin_inff();
    lsep2 = -__builtin_inff();
    if (eqc >= 0) {
      lse2 = a.lse[(size_t)eqc * a.hq + g * G + col % G] * 1.4426950408889634f;
      lsep2 = pa.lsep[(size_t)eqc * a.hkv + g] * 1.4426950408889634f;
    }
  };
  auto store_slot = [&](int slot, const u32x4 qv[2], const u32x4& pv) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      *reinterpret_cast<u32x4*>(qt[slot] + sw(tid / 16 + 16 * k, 8 * (tid % 16))) = qv[k];
    if (tid < 4 * DP)
      *reinterpret_cast<u32x4*>(qit[slot] + (tid / (DP / 8)) * DP + 8 * (tid % (DP / 8))) = pv;
  };

  TileIt it{0, 0, 0, 0};
  bool have = next_segment(a, s, g, b, lo, hi, it);
  int cur_et = it.et, cur_e1 = it.e1;
  int eq[2] = {-1, -1}, eqi = -1, eqc = -1;
  u32x4 qv[2], pv;
  float lse2 = 0.f, lsep2 = 0.f;
  if (have) {
    load_rows(cur_et, cur_e1, eq, eqi, eqc);
    load_data(eq, eqi, eqc, qv, pv, lse2, lsep2);
    store_slot(0, qv, pv);
  }
  int cur_t = eqc;
  it.et += TE;
  bool have_next = have && (it.et < it.e1 || next_segment(a, s, g, b, lo, hi, it));
  int slot = 0;
  while (have) {
    __syncthreads();                         // slot written; last tile's reads done
    const int nx_et = it.et, nx_e1 = it.e1;
    int nq[2] = {-1, -1}, nqi = -1, nqc = -1;
    if (have_next) load_rows(nx_et, nx_e1, nq, nqi, nqc);
    const bool row_ok = cur_t >= 0;
    const int pos = sq.nk - sq.nq + (cur_t - sq.q0);

    f32x16 st = {}, zt = {};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
      st = mfma32(kf[ks], read_rows_sw(qt[slot], 0, 16 * ks, lane), st);
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks)
      zt = mfma32(kif[ks], read_rows(qit[slot], DP, 0, 16 * ks, lane), zt);
    uint16_t* const zb = zbuf[wave];
    // the row's visible keys among the wave's: key0 + m with m <= kmax (in the sequence and,
    // causal, not after the query; none for a padding row or a row without visible keys)
    int kmax = min(kBlock - 1, sq.nk - 1 - u0) - key0;
    if (a.causal) kmax = min(kmax, pos - u0 - key0);
    if (!(row_ok && lse2 > -__builtin_inff() && lsep2 > -__builtin_inff())) kmax = -1;
    const float c1 = pa.pscale * (1.f / G), c2 = pa.pscale * (1.f / (G * G));
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = 8 * q4 + 4 * hf + i <= kmax;
        float p = vis ? __builtin_amdgcn_exp2f(fmaf(st[4 * q4 + i], a.scale_log2, -lse2)) : 0.f;
        p = lane_group_sum<G>(p);            // sum over the entry's heads (DPP network)
        const float pp =
            vis ? __builtin_amdgcn_exp2f(fmaf(zt[4 * q4 + i], pa.pscale_log2, -lsep2)) : 0.f;
        d[i] = fmaf(c1, pp, -c2 * p);        // tau_p (Pp - T) / G, T = p / G
      }
      u32x2 w;
      w[0] = pack_bf16x2(d[0], d[1]);
      w[1] = pack_bf16x2(d[2], d[3]);
      *reinterpret_cast<u32x2*>(zb + pswz(col, 8 * q4 + 4 * hf)) = w;
    }
    if (have_next) load_data(nq, nqi, nqc, qv, pv, lse2, lsep2);
    __syncthreads();                         // dz of every wave written
    // dk_idx += (dz / G)^T q_idx over the tile's 32 rows (each entry counted G times)
#pragma unroll
    for (int kr = 0; kr < 2; ++kr) {
      const bf16x8 za = read_tr_p(zb, 16 * kr, 0, lane);
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt)
        acc[dt] = mfma32(za, read_tr(qit[slot], DP, 16 * kr, 32 * dt, lane), acc[dt]);
    }
    // dq_idx of the tile's entries, dims 32 wave .. +31, over all 128 keys
    if (wave < DP / 32) {
      f32x16 dq = {};
#pragma unroll
      for (int kk = 0; kk < kBlock / 16; ++kk)
        dq = mfma32(read_rows_p(zbuf[kk >> 1], 16 * (kk & 1), lane),
                    read_tr(kib, DP, 16 * kk, 32 * wave, lane), dq);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int n = 8 * (rr / 4) + 4 * hf + rr % 4;
        const int e = cur_et + n / G;
        if (n % G == 0 && e < cur_e1)
          __builtin_nontemporal_store(dq[rr] * G, pa.dqi_part + (size_t)e * DP + 32 * wave + col);
      }
    }
    if (have_next) store_slot(slot ^ 1, qv, pv);
    slot ^= 1;
    have = have_next;
    cur_et = nx_et;
    cur_e1 = nx_e1;
    cur_t = nqc;
    if (have) {
      it.et += TE;
      have_next = it.et < it.e1 || next_segment(a, s, g, b, lo, hi, it);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int m = key0 + 8 * (rr / 4) + 4 * hf + rr % 4;
    const int u = u0 + m;
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      if (split)
        __builtin_nontemporal_store(acc[dt][rr], pa.dki_part + ((size_t)chunk * kBlock + m) * DP + 32 * dt + col);
      else if (u < sq.nk)
        pa.dk_idx[((size_t)(sq.k0 + u) * a.hkv + g) * DP + 32 * dt + col] = acc[dt][rr];
    }
  }
}

// dk_idx of split columns: chunk partials added in chunk order.
template <int DP>
__global__ __launch_bounds__(256) void proxy_dk_reduce_kernel(ProxyArgs pa) {
  const BwdArgs& a = pa.b;
  const int cl = blockIdx.x, tid = threadIdx.x;
  const int c0 = a.chunk_base[cl], c1 = a.chunk_base[cl + 1];
  if (c1 - c0 < 2) return;
  const int b = cl % a.nb_max, g = (cl / a.nb_max) % a.hkv, s = cl / (a.nb_max * a.hkv);
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  for (int i = tid; i < kBlock * DP / 4; i += 256) {
    const int m = i / (DP / 4), u = b * kBlock + m;
    if (u >= sq.nk) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = c0; c < c1; ++c)
      acc += reinterpret_cast<const f32x4*>(pa.dki_part + (size_t)c * kBlock * DP)[i];
    reinterpret_cast<f32x4*>(pa.dk_idx + ((size_t)(sq.k0 + u) * a.hkv + g) * DP)[i % (DP / 4)] =
        acc;
  }
}

// dq_idx[t, g] = sum over the (query, group)'s entries of their partials.
__global__ __launch_bounds__(256) void proxy_dq_kernel(const int32_t* __restrict__ cmap,
                                                       const float* __restrict__ part,
                                                       float* __restrict__ dq, int64_t n,
                                                       int dp, int topk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % (dp / 4));
  const int64_t row = i / (dp / 4);          // query row * hkv + group
  const int32_t* cm = cmap + row * topk;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < topk; ++k) {
    const int e = cm[k];
    if (e >= 0) acc += *reinterpret_cast<const f32x4*>(part + (size_t)e * dp + 4 * c);
  }
  *reinterpret_cast<f32x4*>(dq + row * dp + 4 * c) = acc;
}

template <int G>
hipError_t launch_kv_g(const BwdArgs& a, int64_t chunks_max, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kv_kernel<G>), dim3((unsigned)chunks_max), dim3(512), 0, st, a);
  return hipGetLastError();
}

// Rows (query heads) per chunk of a column; a chunk is 128 tiles of 32 rows.
constexpr int kChunkRows = 4096;

struct BwdGeometry {
  int64_t n_cols, chunks_max;
  size_t off_dq, off_base, off_col, off_kv, total;
};

BwdGeometry bwd_geometry(const msa_shape& s) {
  const Geometry g = geometry(s, MSA_KV_OUTER);
  const Layout L = layout(s, MSA_KV_OUTER);
  BwdGeometry b;
  b.n_cols = (int64_t)s.batch * s.hkv * g.nb_max;
  b.chunks_max = g.e_max / (kChunkRows / g.group) + b.n_cols;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  b.off_dq = take((size_t)g.e_max * g.group * kD * 2);
  b.off_base = take((size_t)(b.n_cols + 1) * 4);
  b.off_col = take((size_t)b.chunks_max * 4);
  b.off_kv = take((size_t)b.chunks_max * 2 * kBlock * kD * 4);
  b.total = off;
  return b;
}

struct ProxyGeometry {
  int64_t n_cols, chunks_max;
  size_t off_dqi, off_base, off_col, off_dki, off_lsep, off_pm, off_pl, total;
};

ProxyGeometry proxy_geometry(const msa_shape& s) {
  const Geometry g = geometry(s, MSA_KV_OUTER);
  const Layout L = layout(s, MSA_KV_OUTER);
  ProxyGeometry b;
  b.n_cols = (int64_t)s.batch * s.hkv * g.nb_max;
  b.chunks_max = g.e_max / (kChunkRows / g.group) + b.n_cols;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  b.off_dqi = take((size_t)g.e_max * s.dp * 4);
  b.off_base = take((size_t)(b.n_cols + 1) * 4);
  b.off_col = take((size_t)b.chunks_max * 4);
  b.off_dki = take((size_t)b.chunks_max * kBlock * s.dp * 4);
  b.off_lsep = take((size_t)s.total_q * s.hkv * 4);
  b.off_pm = take((size_t)g.e_max * 4);
  b.off_pl = take((size_t)g.e_max * 4);
  b.total = off;
  return b;
}

template <int G, int DP>
hipError_t launch_proxy_g(const ProxyArgs& pa, int64_t chunks_max, hipStream_t st) {
  hipLaunchKernelGGL((proxy_bwd_kernel<G, DP>), dim3((unsigned)chunks_max), dim3(256), 0, st, pa);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_proxy_dp(const ProxyArgs& pa, int group, int64_t chunks_max, hipStream_t st) {
  switch (group) {
    case 1: return launch_proxy_g<1, DP>(pa, chunks_max, st);
    case 2: return launch_proxy_g<2, DP>(pa, chunks_max, st);
    case 4: return launch_proxy_g<4, DP>(pa, chunks_max, st);
    case 8: return launch_proxy_g<8, DP>(pa, chunks_max, st);
    default: return launch_proxy_g<16, DP>(pa, chunks_max, st);
  }
}

}  // namespace

size_t proxy_bwd_workspace_bytes(const msa_shape& s) { return proxy_geometry(s).total; }

hipError_t launch_proxy_bwd(const msa_shape& s, const void* q, const void* k, const void* q_idx,
                            const void* k_idx, const float* lse, float scale, float proxy_scale,
                            const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k,
                            char* ws, float* dq_idx, float* dk_idx, float* lse_proxy,
                            hipStream_t st) {
  const Geometry g = geometry(s, MSA_KV_OUTER);
  const Layout L = layout(s, MSA_KV_OUTER);
  const ProxyGeometry pg = proxy_geometry(s);
  if (s.total_k == 0 && s.total_q == 0) return hipSuccess;
  const int64_t n_map = (int64_t)s.total_q * s.hkv * s.topk;
  if (n_map > 0)
    hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)((n_map + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(ws + L.cmap), n_map);
  hipError_t e = launch_plan(s, g, L, lists, cu_q, cu_k, ws, st);
  if (e != hipSuccess) return e;
  ProxyArgs pa{};
  BwdArgs& a = pa.b;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  a.entry_q = reinterpret_cast<const int32_t*>(ws + L.entry_q);
  a.chunk_base = reinterpret_cast<const int32_t*>(ws + pg.off_base);
  a.col_of = reinterpret_cast<const int32_t*>(ws + pg.off_col);
  a.chunk_e = kChunkRows / g.group;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.nb_max = (int)g.nb_max;
  a.wr = (int)g.wr;
  a.n_r = (int)g.n_r;
  a.causal = s.causal;
  pa.q_idx = (const uint16_t*)q_idx;
  pa.k_idx = (const uint16_t*)k_idx;
  float* const lsep = lse_proxy ? lse_proxy : reinterpret_cast<float*>(ws + pg.off_lsep);
  pa.lsep = lsep;
  pa.dqi_part = reinterpret_cast<float*>(ws + pg.off_dqi);
  pa.dki_part = reinterpret_cast<float*>(ws + pg.off_dki);
  pa.dk_idx = dk_idx;
  pa.pscale = proxy_scale;
  pa.pscale_log2 = proxy_scale * 1.4426950408889634f;
  float* const pm = reinterpret_cast<float*>(ws + pg.off_pm);
  float* const pl = reinterpret_cast<float*>(ws + pg.off_pl);
  if (pg.n_cols > 0) {
    hipLaunchKernelGGL(bwd_chunks_kernel, dim3(1), dim3(256), 0, st, a,
                       reinterpret_cast<int32_t*>(ws + pg.off_base),
                       reinterpret_cast<int32_t*>(ws + pg.off_col), (int)pg.n_cols,
                       (int)pg.chunks_max);
    if (s.dp == 32)
      hipLaunchKernelGGL(proxy_lse_part_kernel<32>, dim3((unsigned)pg.chunks_max), dim3(256), 0,
                         st, pa, pm, pl);
    else
      hipLaunchKernelGGL(proxy_lse_part_kernel<64>, dim3((unsigned)pg.chunks_max), dim3(256), 0,
                         st, pa, pm, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)s.total_q * s.hkv;
  if (rows > 0) {
    hipLaunchKernelGGL(proxy_lse_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       st, reinterpret_cast<const int32_t*>(ws + L.cmap),
                       reinterpret_cast<const int32_t*>(ws + L.counters), pm, pl, lsep, rows,
                       s.topk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pg.n_cols > 0) {
    e = s.dp == 32 ? launch_proxy_dp<32>(pa, g.group, pg.chunks_max, st)
                   : launch_proxy_dp<64>(pa, g.group, pg.chunks_max, st);
    if (e != hipSuccess) return e;
    if (s.dp == 32)
      hipLaunchKernelGGL(proxy_dk_reduce_kernel<32>, dim3((unsigned)pg.n_cols), dim3(256), 0, st,
                         pa);
    else
      hipLaunchKernelGGL(proxy_dk_reduce_kernel<64>, dim3((unsigned)pg.n_cols), dim3(256), 0, st,
                         pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = (int64_t)s.total_q * s.hkv * (s.dp / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(proxy_dq_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const int32_t*>(ws + L.cmap), pa.dqi_part, dq_idx, n, s.dp,
                     s.topk);
  return hipGetLastError();
}

size_t bwd_workspace_bytes(const msa_shape& s) { return bwd_geometry(s).total; }

bool bwd_fits(const msa_shape& s) {
  const BwdGeometry b = bwd_geometry(s);
  if (proxy_geometry(s).chunks_max != b.chunks_max) return false;
  return b.chunks_max < (1LL << 31) && b.n_cols + 1 < (1LL << 31);
}

hipError_t launch_bwd(const msa_shape& s, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, float scale,
                      const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k, char* ws,
                      float* dq, float* dk, float* dv, hipStream_t st) {
  const Geometry g = geometry(s, MSA_KV_OUTER);
  const Layout L = layout(s, MSA_KV_OUTER);
  if (s.total_k == 0 && s.total_q == 0) return hipSuccess;
  const int64_t n_map = (int64_t)s.total_q * s.hkv * s.topk;
  if (n_map > 0)
    hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)((n_map + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(ws + L.cmap), n_map);
  hipError_t e = launch_plan(s, g, L, lists, cu_q, cu_k, ws, st);
  if (e != hipSuccess) return e;
  float* const dsum = reinterpret_cast<float*>(ws + L.part_lse);   // [total_q, hq]
  const int rows = s.total_q * s.hq;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                       (const uint16_t*)o, (const uint16_t*)dout, dsum, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.dsum = dsum;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.offsets = reinterpret_cast<const int32_t*>(ws + L.offsets);
  a.entry_q = reinterpret_cast<const int32_t*>(ws + L.entry_q);
  const BwdGeometry bg = bwd_geometry(s);
  a.dq_part = reinterpret_cast<uint16_t*>(ws + bg.off_dq);
  a.chunk_base = reinterpret_cast<const int32_t*>(ws + bg.off_base);
  a.col_of = reinterpret_cast<const int32_t*>(ws + bg.off_col);
  a.dkv_part = reinterpret_cast<float*>(ws + bg.off_kv);
  a.chunk_e = kChunkRows / g.group;
  a.dk = dk;
  a.dv = dv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.total_q = s.total_q;
  a.total_k = s.total_k;
  a.max_q = s.max_q;
  a.max_k = s.max_k;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.nb_max = (int)g.nb_max;
  a.wr = (int)g.wr;
  a.n_r = (int)g.n_r;
  a.causal = s.causal;
  if (bg.n_cols > 0) {
    hipLaunchKernelGGL(bwd_chunks_kernel, dim3(1), dim3(256), 0, st, a,
                       reinterpret_cast<int32_t*>(ws + bg.off_base),
                       reinterpret_cast<int32_t*>(ws + bg.off_col), (int)bg.n_cols,
                       (int)bg.chunks_max);
    switch (g.group) {
      case 1: e = launch_kv_g<1>(a, bg.chunks_max, st); break;
      case 2: e = launch_kv_g<2>(a, bg.chunks_max, st); break;
      case 4: e = launch_kv_g<4>(a, bg.chunks_max, st); break;
      case 8: e = launch_kv_g<8>(a, bg.chunks_max, st); break;
      default: e = launch_kv_g<16>(a, bg.chunks_max, st); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_kv_reduce_kernel, dim3((unsigned)bg.n_cols, kReduceParts), dim3(256), 0,
                       st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = (int64_t)rows * 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const int32_t*>(ws + L.cmap), a.dq_part, dq, n, s.hq,
                     g.group, s.topk);
  return hipGetLastError();
}

}  // namespace msa
