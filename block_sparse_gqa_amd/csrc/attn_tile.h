// One 128-key block of attention for up to 32 query rows per wave, on bf16 MFMA.
//
// The block's K (row = key) and V^T (row = head dim) live in LDS as 128 rows of 256 bytes
// with 16-byte chunks XOR-swizzled by swz(row). A wave owns 32 rows (one per lane column):
//   S^T[key][row] = sum_d K[key][d] Q[row][d]        (A = K from LDS, B = Q from registers)
//   O^T[dim][row] += sum_key V^T[dim][key] P[row][key] (A = V^T from LDS, B = P in registers)
// Lane l holds keys 32*kt + 16*(l/32) + r of its row in s[kt][r], and dims
// 32*dt + 16*(l/32) + r in o[dt][r].
#pragma once
#include "msa_device.h"

namespace msa {

struct KVLds {
  u32x4 k[128 * 16];
  u32x4 vt[128 * 16];
};

// Stage block rows [u0, u0 + 128) of one KV head into LDS. Rows at or past `nk_rel` (keys
// past the end of the sequence) are zero. `row_stride`: elements between consecutive keys
// (127 * row_stride must fit in 32 bits, i.e. hkv * d < 2^24). 256 threads.
template <bool FP8>
__device__ __forceinline__ void stage_kv(KVLds& L, const void* kbase, const void* vbase,
                                         uint32_t row_stride, int nk_rel) {
  // Opaque copy of the thread id: keeps the compiler from hoisting the 16 per-thread row
  // offsets out of the caller's loops (they would stay live, or spill, for the whole kernel).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  if constexpr (!FP8) {
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(kbase);
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(vbase);
    // K: 2048 chunks of 16 B, 8 per thread; 16 consecutive threads read one row.
    u32x4 kr[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int i = tid + 256 * p;
      const int row = i >> 4, cc = i & 15;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < nk_rel) v = *reinterpret_cast<const u32x4*>(kp + (uint32_t)row * row_stride + cc * 8);
      kr[p] = v;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int i = tid + 256 * p;
      const int row = i >> 4, cc = i & 15;
      L.k[row * 16 + (cc ^ swz(row))] = kr[p];
    }
    // V: thread owns keys 8*kg..+7 and dims 8*dg..+7, transposed in registers.
    const int kg = tid >> 4, dg = tid & 15;
    u32x4 vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * kg + i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < nk_rel) v = *reinterpret_cast<const u32x4*>(vp + (uint32_t)row * row_stride + dg * 8);
      vr[i] = v;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = vr[2 * q][j >> 1], b = vr[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      const int row = 8 * dg + j;
      L.vt[row * 16 + (kg ^ swz(row))] = o;
    }
  } else {
    const uint8_t* kp = reinterpret_cast<const uint8_t*>(kbase);
    const uint8_t* vp = reinterpret_cast<const uint8_t*>(vbase);
    // K: 1024 chunks of 16 fp8 (= 2 bf16 chunks), 4 per thread.
    u32x4 kr[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = tid + 256 * p;
      const int row = i >> 3, c8 = i & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < nk_rel) v = *reinterpret_cast<const u32x4*>(kp + (uint32_t)row * row_stride + c8 * 16);
      kr[p] = v;
    }
    const int kg = tid >> 4, dg = tid & 15;
    u32x2 vr8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * kg + i;
      u32x2 v = {0u, 0u};
      if (row < nk_rel) v = *reinterpret_cast<const u32x2*>(vp + (uint32_t)row * row_stride + dg * 8);
      vr8[i] = v;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = tid + 256 * p;
      const int row = i >> 3, c8 = i & 7;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const u32x2 lo = fp8x4_to_bf16x4(kr[p][2 * hlf]);
        const u32x2 hi = fp8x4_to_bf16x4(kr[p][2 * hlf + 1]);
        u32x4 o = {lo[0], lo[1], hi[0], hi[1]};
        const int cc = 2 * c8 + hlf;
        L.k[row * 16 + (cc ^ swz(row))] = o;
      }
    }
    u32x4 vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x2 lo = fp8x4_to_bf16x4(vr8[i][0]);
      const u32x2 hi = fp8x4_to_bf16x4(vr8[i][1]);
      vr[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = vr[2 * q][j >> 1], b = vr[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
      }
      const int row = 8 * dg + j;
      L.vt[row * 16 + (kg ^ swz(row))] = o;
    }
  }
}

// B operand of S^T: the lane's Q row, d = 16*st + 8*(l/32) + i in bq[st]. The loads are
// unconditional (padding rows point at a valid row), which keeps them free of exec-masked
// branches so the compiler can leave them in flight across a whole tile of work.
template <bool FP8>
__device__ __forceinline__ void load_q_operand(bf16x8 bq[8], const void* qrow, int hf) {
  if constexpr (!FP8) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(qrow);
#pragma unroll
    for (int st = 0; st < 8; ++st)
      bq[st] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + 16 * st + 8 * hf));
  } else {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(qrow);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p + 16 * st + 8 * hf);
      const u32x2 lo = fp8x4_to_bf16x4(v[0]);
      const u32x2 hi = fp8x4_to_bf16x4(v[1]);
      bq[st] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  }
}

// S^T for the wave's 32 rows over the block's 128 keys: 32 MFMAs. The K operands of step
// st+1 are read from LDS while the MFMAs of step st run.
__device__ __forceinline__ void qk_block(const KVLds& L, const bf16x8 bq[8], f32x16 s[4],
                                         int col, int hf) {
  const int rp = rowperm(col);
  const int sw = swz(rp);                 // swz(32*kt + rp) == swz(rp)
  bf16x8 a[2][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) a[0][kt] = as_bf16x8(L.k[(kt * 32 + rp) * 16 + (hf ^ sw)]);
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    if (st + 1 < 8) {
      const int cc = (2 * (st + 1) + hf) ^ sw;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) a[(st + 1) & 1][kt] = as_bf16x8(L.k[(kt * 32 + rp) * 16 + cc]);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      s[kt] = mfma32(a[st & 1][kt], bq[st], st == 0 ? f32x16{} : s[kt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T (+)= V^T P^T over the block: 32 MFMAs; p holds the row's probabilities as packed
// bf16 pairs, p[kt][ks][i] = keys 32*kt + 16*(l/32) + 8*ks + 2i, +1. With `init`, o starts
// from zero instead of accumulating.
template <bool INIT>
__device__ __forceinline__ void pv_block(const KVLds& L, const u32x4 p[4][2], f32x16 o[4],
                                         int col, int hf) {
  const int rp = rowperm(col);
  const int sw = swz(rp);                 // swz(32*dt + rp) == swz(rp)
#pragma unroll
  for (int step = 0; step < 8; ++step) {
    const int kt = step >> 1, ks = step & 1;
    const int cc = (4 * kt + 2 * hf + ks) ^ sw;
    bf16x8 a[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) a[dt] = as_bf16x8(L.vt[(dt * 32 + rp) * 16 + cc]);
    const bf16x8 bp = as_bf16x8(p[kt][ks]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      o[dt] = mfma32(a[dt], bp, (INIT && step == 0) ? f32x16{} : o[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- row-major staging by direct-to-LDS loads (bf16), for pipelined block loops
// K keeps the layout above (chunk c of key row r at slot c ^ swz(r)); V is stored row-major
// too, chunk c of key row r at slot c ^ swz_v(r), and read transposed with the LDS transpose
// load. swz_v depends on r % 4 only, so every transposed read of a lane is its fixed base
// address plus a compile-time offset.
__device__ __forceinline__ int swz_v(int key) { return (key & 3) << 2; }

// s_waitcnt vmcnt(n): direct-to-LDS loads are not tracked by the compiler's own waits.
// The count has 6 bits: bits 3:0 of the immediate and bits 15:14.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// 16 bytes per lane from global memory to LDS address `lds` + 16 * lane (`lds` wave-uniform),
// as inline assembly. The compiler does not see these loads, so it adds no wait for them before
// later LDS reads: with the builtin it waits for every direct-to-LDS load in flight, the next
// block's included, before the first LDS read of the current block, which serialises the
// prefetch with the math. The caller makes the data visible (wait_vm<n>() and a barrier).
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a)
               : "memory", "m0");
}

// Marks the Q operand as used at this point. Called right after the caller has waited for
// every load in flight, it places the compiler's own wait for the Q loads there instead of at
// the first MFMA, which comes after the next block's loads have been issued (the compiler's
// wait counts only the loads it knows of, so it would wait for those too).
__device__ __forceinline__ void hold_q(bf16x8 bq[8]) {
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" : "+v"(bq[st]));
}

// One 128-row x 256-byte block (rows at or past nk_rel repeat row nk_rel - 1; the caller masks
// or zero-weights them) into `dst` by 256 threads t = 0..255, 8 loads each: slot i of the block holds chunk
// (i % 16) ^ f(i / 16) of row i / 16, lane l fetching exactly the chunk its slot needs.
template <bool V>
__device__ __forceinline__ void dma_rows_t(u32x4* dst, const uint16_t* base, uint32_t row_stride,
                                           int nk_rel, int t) {
  asm volatile("" : "+v"(t));
  const int wave = t >> 6, row0 = t >> 4, slot = t & 15;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int row = 16 * p + row0;        // swz(row) and swz_v(row) from row0 and p
    const int f = V ? swz_v(row0)
                    : ((row0 & 3) | ((p & 1) << 2) | (((row0 >> 2) & 1) << 3));
    const uint32_t r = (uint32_t)min(row, nk_rel - 1);
    lds_dma16(base + r * row_stride + (uint32_t)((slot ^ f) * 8), dst + p * 256 + wave * 64);
  }
}

// The same with the workgroup's own 256 threads (thread t = threadIdx.x).
template <bool V>
__device__ __forceinline__ void dma_rows(u32x4* dst, const uint16_t* base, uint32_t row_stride,
                                         int nk_rel) {
  dma_rows_t<V>(dst, base, row_stride, nk_rel, (int)threadIdx.x);
}

// ---- half blocks: a wave covering keys [32*kt0, 32*kt0 + 64) of a staged block

// S^T for the wave's 32 rows over keys 32*kt0 .. +63 of the block in `kb` (K layout above):
// 16 MFMAs, s[i] holding keys 32*(kt0 + i) + 16*(l/32) + r. The K operands are read two
// steps ahead of their MFMAs (a ring of three steps), so a caller can spread other work
// between the MFMAs without waiting on LDS.
__device__ __forceinline__ void qk_half(const u32x4* kb, const bf16x8 bq[8], f32x16 s[2],
                                        int kt0, int col, int hf) {
  const int rp = rowperm(col);
  const int sw = swz(rp);                 // swz(32*kt + rp) == swz(rp)
  const u32x4* r0 = kb + (kt0 * 32 + rp) * 16;
  bf16x8 a[3][2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int cc = (2 * st + hf) ^ sw;
    a[st][0] = as_bf16x8(r0[cc]);
    a[st][1] = as_bf16x8(r0[32 * 16 + cc]);
  }
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    if (st + 2 < 8) {
      const int cc = (2 * (st + 2) + hf) ^ sw;
      a[(st + 2) % 3][0] = as_bf16x8(r0[cc]);
      a[(st + 2) % 3][1] = as_bf16x8(r0[32 * 16 + cc]);
    }
    s[0] = mfma32(a[st % 3][0], bq[st], st == 0 ? f32x16{} : s[0]);
    s[1] = mfma32(a[st % 3][1], bq[st], st == 0 ? f32x16{} : s[1]);
  }
}

// O^T += V^T P^T over keys 32*kt0 .. +63 of the row-major V block in `vb` (layout of
// dma_rows<true>): 16 MFMAs; p[i][ks] holds keys 32*(kt0 + i) + 16*(l/32) + 8*ks + 2j, +1.
// The LDS transpose load gives lane j of each 16-lane group elements from the 16 rows x 4
// columns its group's lanes address: lane s of the group addresses key row k0 + s/4 at dims
// D(s%4) .. +3 with D = {0, 16, 4, 20} (+8 for the group of lanes 16..31), and lane j receives
// dims D(j/4) + j%4 = rowperm(j) of keys k0 .. k0+3, i.e. its A-operand row for four
// consecutive keys.
__device__ __forceinline__ void pv_half_tr(const u32x4* vb, const u32x4 p[2][2], f32x16 o[4],
                                           int kt0, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  asm volatile("" : "+v"(lane));
  const int s = lane & 15, grp = (lane >> 4) & 1, hf = lane >> 5;
  const int dsel = s & 3, k_lane = s >> 2;
  const int d_lane = ((dsel & 1) << 4) + ((dsel >> 1) << 2) + 8 * grp;
  const unsigned short* vrow = reinterpret_cast<const unsigned short*>(vb) + kt0 * 32 * 128;
  const unsigned short* base[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    base[dt] = vrow + (16 * hf + k_lane) * 128 + (4 * (dt ^ k_lane) + (d_lane >> 3)) * 8 +
               (d_lane & 7);
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int kt = step >> 1, ks = step & 1;
    bf16x8 a[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      s4 r[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        r[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(base[dt] + (32 * kt + 8 * ks + 4 * h2) * 128));
      a[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const bf16x8 bp = as_bf16x8(p[kt][ks]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(a[dt], bp, o[dt]);
  }
}

// Row max of raw scores over the block, keys past `kmax` (block-relative index of the last
// visible key) set to -inf first when `need_mask`. Both lanes of the row agree.
__device__ __forceinline__ float mask_max(f32x16 s[4], int kmax, bool need_mask, int hf) {
  const float ninf = -__builtin_inff();
  if (need_mask) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[kt][r] = (kt * 32 + 16 * hf + r <= kmax) ? s[kt][r] : ninf;
  }
  float m = ninf;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kt][r]);
  return fmaxf(m, shfl_xor_f(m, 32));
}

// p = 2^(s * sl2 - c) packed to bf16 pairs; returns the fp32 row sum (both lanes agree).
// c = row max * sl2 (finite); masked scores (-inf) give 0.
__device__ __forceinline__ float exp_pack(const f32x16 s[4], float sl2, float c, u32x4 p[4][2]) {
  float l = 0.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * ks + 2 * i], sl2, -c));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * ks + 2 * i + 1], sl2, -c));
        l += x0 + x1;
        p[kt][ks][i] = pack_bf16x2(x0, x1);
      }
    }
  }
  return l + shfl_xor_f(l, 32);
}

// Row max of raw scores over the wave's half block (s[i]: block keys 32*(kt0 + i) + 16*(l/32)
// + r), keys past `kmax` (block-relative) set to -inf first when `need_mask`.
__device__ __forceinline__ float mask_max_half(f32x16 s[2], int kt0, int kmax, bool need_mask,
                                               int hf) {
  const float ninf = -__builtin_inff();
  if (need_mask) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[i][r] = ((kt0 + i) * 32 + 16 * hf + r <= kmax) ? s[i][r] : ninf;
  }
  float m = ninf;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, s[i][r]);
  return fmaxf(m, shfl_xor_f(m, 32));
}

// p = 2^(s * sl2 - c) over the half block as packed bf16 pairs; returns this lane's sum of
// the rounded p (the row's other 32 keys sit in lane l ^ 32).
__device__ __forceinline__ float exp_pack_half(const f32x16 s[2], float sl2, float c,
                                               u32x4 p[2][2]) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[i][8 * ks + 2 * j], sl2, -c));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[i][8 * ks + 2 * j + 1], sl2, -c));
        const uint32_t w = pack_bf16x2(x0, x1);
        p[i][ks][j] = w;
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l, false);
      }
  return l;
}

// Pack 16 consecutive output dims per dt (scaled by `mul`) as bf16: w[2*dt + h2] holds dims
// 32*dt + 16*(l/32) + 8*h2 .. +8.
__device__ __forceinline__ void pack_o_row(u32x4 w[8], const f32x16 o[4], float mul) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[2 * dt + h2][i] = pack_bf16x2(o[dt][8 * h2 + 2 * i] * mul, o[dt][8 * h2 + 2 * i + 1] * mul);
}

__device__ __forceinline__ void store_packed_row(uint16_t* orow, const u32x4 w[8], int hf) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<u32x4*>(orow + (j >> 1) * 32 + 16 * hf + 8 * (j & 1)) = w[j];
}

// Write 16 consecutive output dims per dt (scaled by `mul`) as bf16 to orow[0..128).
__device__ __forceinline__ void store_o_row(uint16_t* orow, const f32x16 o[4], float mul, int hf) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(o[dt][8 * h2 + 2 * i] * mul, o[dt][8 * h2 + 2 * i + 1] * mul);
      *reinterpret_cast<u32x4*>(orow + dt * 32 + 16 * hf + 8 * h2) = w;
    }
  }
}

// The same row as a partial output (row p of the partial buffer, 8-row group layout).
__device__ __forceinline__ void store_o_part(uint16_t* part_o, size_t p, const f32x16 o[4],
                                             float mul, int hf) {
  char* const base = reinterpret_cast<char*>(part_o);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(o[dt][8 * h2 + 2 * i] * mul, o[dt][8 * h2 + 2 * i + 1] * mul);
      *reinterpret_cast<u32x4*>(base + part_chunk_offset(p, 4 * dt + 2 * hf + h2)) = w;
    }
  }
}

}  // namespace msa
