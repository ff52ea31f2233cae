// Device-side building blocks shared by the gfx950 kernels of libmsa.
//
// MFMA operand layout used throughout (v_mfma_f32_32x32x16_bf16, wave64): for
// D[m][n] = sum_k A[m][k] * B[k][n], lane l supplies A[l%32][8*(l/32) + i] and
// B[8*(l/32) + i][l%32] for i = 0..7, and receives D[8*(r/4) + 4*(l/32) + r%4][l%32] in
// accumulator register r = 0..15.
//
// Attention tiles are computed transposed, S^T = K Q^T and O^T = V^T P^T, so that every lane
// owns one query row (column l%32) and a row's softmax needs a single cross-lane exchange
// (lane l with lane l^32). Rows of the K and V^T operands are fed in the order ROWPERM so
// that lane l holds 16 consecutive keys (or output dims) 16*(l/32) + r in register r.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;      // KV block (tokens)
constexpr int kD = 128;          // head dim
constexpr int kMaxTopK = 16;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Output row m of a 32x32 tile -> the key / dim it stands for, so that lane l ends up with
// 16*(l/32) + r in accumulator register r.
__device__ __forceinline__ int rowperm(int m) {
  return (((m >> 2) & 1) << 4) | ((m >> 3) << 2) | (m & 3);
}

// XOR swizzle of 16-byte chunks in a 256-byte LDS row, chosen so that the 16 rows one
// 16-lane group reads (rows rowperm(0..15) or rowperm(16..31) of a 32-row tile) fall on 16
// distinct chunk positions.
__device__ __forceinline__ int swz(int row) {
  return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two round-to-nearest-even bf16 in one dword (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// OCP fp8 e4m3fn byte -> float (exact). Subnormals at exponent 0; 0x7f/0xff are NaN.
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t b) {
  uint32_t s = (b & 0x80u) << 24;
  uint32_t e = (b >> 3) & 0xFu;
  uint32_t m = b & 0x7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;                 // m/8 * 2^-6
  } else if (e == 15 && m == 7) {
    mag = __builtin_nanf("");
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

// Four fp8 bytes (one dword) -> four bf16 (two dwords), exact (every e4m3fn value is a bf16
// value): the gfx950 scaled pack conversion with scale 1. Checked on the device against
// fp8e4m3_to_f32 for all 256 codes in every byte position (NaN codes stay NaN).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ int shfl_xor_i(int v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Cross-lane moves on the DPP network (no LDS traffic). gfx9 controls: quad_perm [1,0,3,2]
// (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), row_half_mirror (lane i of 8 reads 7 - i: the
// other quad), row_mirror (lane i of 16 reads 15 - i: the other half row).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16); every lane gets its group's sum.
// Each level adds the other half of the group, so both halves compute the same sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
  return v;
}

// Max over all 64 lanes of values that are already equal within aligned groups of N lanes.
template <int N>
__device__ __forceinline__ float wave_max_from(float v) {
  if constexpr (N <= 1) v = fmaxf(v, dpp_f<kDppXor1>(v));
  if constexpr (N <= 2) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if constexpr (N <= 4) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N <= 8) v = fmaxf(v, dpp_f<kDppMirror>(v));
  v = fmaxf(v, shfl_xor_f(v, 16));
  return fmaxf(v, shfl_xor_f(v, 32));
}

// Partial outputs (bf16, 256 bytes per row) are stored in groups of 8 rows: chunk c (dims
// 8c .. 8c+7) of partial row p sits at byte ((p / 8) * 16 + c) * 128 + (p % 8) * 16, so chunk
// c of 8 consecutive rows is one 128-byte line. A wave holding whole rows of 8-row groups
// then writes 1 KiB of consecutive bytes per store instruction straight from its MFMA
// registers, and the combine reads an entry of G >= 8 heads as G * 256 consecutive bytes.
__device__ __forceinline__ size_t part_chunk_offset(size_t p, int c) {
  return ((p >> 3) << 11) + ((size_t)c << 7) + ((p & 7) << 4);
}

// Per-sequence geometry read from the cumulative length arrays.
struct Seq {
  int q0, nq, k0, nk;
};

__device__ __forceinline__ Seq load_seq(const int32_t* cu_q, const int32_t* cu_k, int s) {
  Seq r;
  r.q0 = cu_q[s];
  r.nq = cu_q[s + 1] - r.q0;
  r.k0 = cu_k[s];
  r.nk = cu_k[s + 1] - r.k0;
  return r;
}

// Sequence geometry clamped to the tensor extents and the max_q / max_k bounds, so that
// inconsistent length arrays cannot send any kernel outside the caller's buffers.
__device__ __forceinline__ Seq load_seq_clamped(const int32_t* cu_q, const int32_t* cu_k, int s,
                                                int total_q, int total_k, int max_q,
                                                int max_k) {
  Seq r;
  const int q0 = min(max(cu_q[s], 0), total_q);
  const int q1 = min(max(cu_q[s + 1], q0), total_q);
  const int k0 = min(max(cu_k[s], 0), total_k);
  const int k1 = min(max(cu_k[s + 1], k0), total_k);
  r.q0 = q0;
  r.nq = min(q1 - q0, max_q);
  r.k0 = k0;
  r.nk = min(k1 - k0, max_k);
  return r;
}

// Running top list of (score, block) sorted by score descending; a new block goes after
// equal scores, so blocks inserted in ascending order keep the lower index first among ties.
// Fully unrolled so that the list lives in registers.
struct TopList {
  float sc[kMaxTopK];
  int id[kMaxTopK];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) { sc[k] = -__builtin_inff(); id[k] = -1; }
  }
  __device__ __forceinline__ void insert(float v, int j) {
#pragma unroll
    for (int k = kMaxTopK - 1; k >= 1; --k) {
      const bool gp = v > sc[k - 1];
      const bool gc = v > sc[k];
      sc[k] = gp ? sc[k - 1] : (gc ? v : sc[k]);
      id[k] = gp ? id[k - 1] : (gc ? j : id[k]);
    }
    const bool g0 = v > sc[0];
    sc[0] = g0 ? v : sc[0];
    id[0] = g0 ? j : id[0];
  }
};

// (a beats b) in the order score desc, block asc; empty entries (-1) lose to everything.
__device__ __forceinline__ bool beats(float sa, int ia, float sb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return sa > sb || (sa == sb && ia < ib);
}

// floor(a / b) for b > 0 and any sign of a.
__device__ __forceinline__ int floordiv(int a, int b) {
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

}  // namespace msa
