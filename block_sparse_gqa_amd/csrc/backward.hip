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

// D[t, h] = sum_d dO[t, h, d] O[t, h, d] (fp32), one wave per row of 128.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       float* __restrict__ dsum, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint32_t a = reinterpret_cast<const uint32_t*>(o + (size_t)row * kD)[lane];
  const uint32_t b = reinterpret_cast<const uint32_t*>(dout + (size_t)row * kD)[lane];
  float v = bf16_bits_to_f32(a & 0xFFFFu) * bf16_bits_to_f32(b & 0xFFFFu) +
            bf16_bits_to_f32(a >> 16) * bf16_bits_to_f32(b >> 16);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += shfl_xor_f(v, off);
  if (lane == 0) dsum[row] = v;
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
  float* dq_part;
  float* dk;
  float* dv;
  float scale, scale_log2;
  int total_q, total_k, max_q, max_k, hq, hkv, nb_max, wr, n_r, causal;
};

template <int G>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdArgs a) {
  constexpr int TE = 32 / G;                 // entries per tile of 32 rows
  __shared__ uint16_t kb[kBlock * kD];       // K_b, V_b, row-major
  __shared__ uint16_t vb[kBlock * kD];
  __shared__ uint16_t qt[32 * kD];           // the tile's Q and dO rows
  __shared__ uint16_t dot[32 * kD];
  __shared__ uint16_t pbuf[4][32 * 32];      // per wave: P and dS of its keys, [row][key]
  __shared__ uint16_t sbuf[4][32 * 32];
  __shared__ float red[4][32][64];           // dQ of the four waves, half the dims at a time

  const int b = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const Seq sq = load_seq_clamped(a.cu_q, a.cu_k, s, a.total_q, a.total_k, a.max_q, a.max_k);
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  if (b >= nb) return;
  const int u0 = b * kBlock;

  // K_b and V_b (rows past the sequence repeat its last key; their weights are masked)
  for (int i = tid; i < kBlock * kD / 8; i += 256) {
    const int row = i / (kD / 8), c = i % (kD / 8);
    const size_t src = ((size_t)(sq.k0 + min(u0 + row, sq.nk - 1)) * a.hkv + g) * kD + 8 * c;
    *reinterpret_cast<u32x4*>(kb + row * kD + 8 * c) = *reinterpret_cast<const u32x4*>(a.k + src);
    *reinterpret_cast<u32x4*>(vb + row * kD + 8 * c) = *reinterpret_cast<const u32x4*>(a.v + src);
  }

  f32x16 dk_acc[4], dv_acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk_acc[dt] = f32x16{};
    dv_acc[dt] = f32x16{};
  }
  const int key0 = 32 * wave;                // this wave's keys within the block

  for (int r = 0; r < a.n_r; ++r) {
    const size_t bk = (((size_t)s * a.hkv + g) * a.n_r + r) * a.nb_max + b;
    const int e0 = a.offsets[bk * a.wr], e1 = a.offsets[(bk + 1) * a.wr];
    for (int et = e0; et < e1; et += TE) {
      __syncthreads();                       // K/V staged; previous tile's buffers free
      // Q and dO rows of the tile: row n = entry et + n / G, head g G + n % G
      for (int i = tid; i < 32 * kD / 8; i += 256) {
        const int n = i / (kD / 8), c = i % (kD / 8);
        const int e = et + n / G;
        u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u};
        if (e < e1) {
          const size_t row = (size_t)a.entry_q[e] * a.hq + g * G + n % G;
          qv = *reinterpret_cast<const u32x4*>(a.q + row * kD + 8 * c);
          dv4 = *reinterpret_cast<const u32x4*>(a.dout + row * kD + 8 * c);
        }
        *reinterpret_cast<u32x4*>(qt + n * kD + 8 * c) = qv;
        *reinterpret_cast<u32x4*>(dot + n * kD + 8 * c) = dv4;
      }
      // this lane's row (column n = col of S^T): its query, LSE and D
      const int e_row = et + col / G;
      const bool row_ok = e_row < e1;
      int t = 0;
      float lse2 = 0.f, dsum = 0.f;
      if (row_ok) {
        t = a.entry_q[e_row];
        const size_t hrow = (size_t)t * a.hq + g * G + col % G;
        lse2 = a.lse[hrow] * 1.4426950408889634f;
        dsum = a.dsum[hrow];
      }
      const int pos = sq.nk - sq.nq + (t - sq.q0);
      __syncthreads();

      // S^T and dP^T for the wave's 32 keys x the tile's 32 rows
      f32x16 st = {}, dpt = {};
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const bf16x8 ka = read_rows(kb, kD, key0, 16 * ks, lane);
        const bf16x8 va = read_rows(vb, kD, key0, 16 * ks, lane);
        const bf16x8 qb = read_rows(qt, kD, 0, 16 * ks, lane);
        const bf16x8 ob = read_rows(dot, kD, 0, 16 * ks, lane);
        st = mfma32(ka, qb, st);
        dpt = mfma32(va, ob, dpt);
      }
      // P = exp(tau S - LSE) on visible keys; dS = P (dP - D); both to the wave's buffers as
      // [row][key] (lane (row col, half hf) holds keys 8 (r / 4) + 4 hf + r % 4 in st[r])
      uint16_t* const pb = pbuf[wave];
      uint16_t* const sb = sbuf[wave];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float p[4], d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 8 * q4 + 4 * hf + i;
          const int u = u0 + key0 + m;
          const bool vis = row_ok && u < sq.nk && !(a.causal && u > pos) &&
                           lse2 > -__builtin_inff();
          p[i] = vis ? __builtin_amdgcn_exp2f(fmaf(st[4 * q4 + i], a.scale_log2, -lse2)) : 0.f;
          d[i] = p[i] * (dpt[4 * q4 + i] - dsum);
        }
        u32x2 pw, sw;
        pw[0] = pack_bf16x2(p[0], p[1]);
        pw[1] = pack_bf16x2(p[2], p[3]);
        sw[0] = pack_bf16x2(d[0], d[1]);
        sw[1] = pack_bf16x2(d[2], d[3]);
        *reinterpret_cast<u32x2*>(pb + col * 32 + 8 * q4 + 4 * hf) = pw;
        *reinterpret_cast<u32x2*>(sb + col * 32 + 8 * q4 + 4 * hf) = sw;
      }
      __syncthreads();                       // P, dS of every wave written

      // dV += P^T dO, dK += dS^T Q: contraction over the tile's 32 rows (2 steps of 16)
#pragma unroll
      for (int kr = 0; kr < 2; ++kr) {
        const bf16x8 pa = read_tr(pb, 32, 16 * kr, 0, lane);   // P^T[key][rows]
        const bf16x8 sa = read_tr(sb, 32, 16 * kr, 0, lane);   // dS^T[key][rows]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 ob = read_tr(dot, kD, 16 * kr, 32 * dt, lane);   // dO[rows][dims]
          const bf16x8 qb = read_tr(qt, kD, 16 * kr, 32 * dt, lane);    // Q[rows][dims]
          dv_acc[dt] = mfma32(pa, ob, dv_acc[dt]);
          dk_acc[dt] = mfma32(sa, qb, dk_acc[dt]);
        }
      }
      // dQ of the tile's rows from this wave's keys: dS[rows][keys] K[keys][dims]
      f32x16 dq[4] = {};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 sa = read_rows(sb, 32, 0, 16 * kk, lane);            // dS[row][keys]
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 kbf = read_tr(kb, kD, key0 + 16 * kk, 32 * dt, lane);  // K[keys][dims]
          dq[dt] = mfma32(sa, kbf, dq[dt]);
        }
      }
      // sum over the four waves and write the entries' partials, half the dims at a time
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            red[wave][8 * (rr / 4) + 4 * hf + rr % 4][32 * d2 + col] = dq[2 * half + d2][rr];
        __syncthreads();
        for (int i = tid; i < 32 * 64; i += 256) {
          const int n = i / 64, dd = i % 64;
          const int e = et + n / G;
          if (e < e1) {
            const float v4 = (red[0][n][dd] + red[1][n][dd]) + (red[2][n][dd] + red[3][n][dd]);
            a.dq_part[((size_t)e * G + n % G) * kD + 64 * half + dd] = v4 * a.scale;
          }
        }
        __syncthreads();
      }
    }
  }
  // dK, dV rows of the wave's keys (D layout: lane l, reg r -> key 8 (r / 4) + 4 (l / 32) +
  // r % 4, dim 32 dt + l % 32)
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int u = u0 + key0 + 8 * (rr / 4) + 4 * hf + rr % 4;
    if (u < sq.nk) {
      const size_t row = ((size_t)(sq.k0 + u) * a.hkv + g) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        a.dk[row + 32 * dt + col] = dk_acc[dt][rr] * a.scale;
        a.dv[row + 32 * dt + col] = dv_acc[dt][rr];
      }
    }
  }
}

// dQ[t, h] = sum over the (query, group)'s entries of their partials (the combine map), one
// thread per 4 dims of a (query, head) row.
__global__ __launch_bounds__(256) void bwd_dq_kernel(const int32_t* __restrict__ cmap,
                                                     const float* __restrict__ dq_part,
                                                     float* __restrict__ dq, int64_t n, int hq,
                                                     int group, int topk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % 32);
  const int64_t row = i / 32;                // query row * hq + head
  const int head = (int)(row % hq), h = head / group, gi = head % group;
  const int64_t t = row / hq;
  const int32_t* cm = cmap + (t * (hq / group) + h) * topk;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < topk; ++k) {
    const int e = cm[k];
    if (e < 0) continue;
    acc += *reinterpret_cast<const f32x4*>(dq_part + ((size_t)e * group + gi) * kD + 4 * c);
  }
  *reinterpret_cast<f32x4*>(dq + row * kD + 4 * c) = acc;
}

// The combine map of rows that lie in no sequence is never written by the plan: clear it.
__global__ __launch_bounds__(256) void bwd_clear_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = -1;
}

template <int G>
hipError_t launch_kv_g(const msa_shape& s, const Geometry& g, const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kv_kernel<G>), dim3((unsigned)g.nb_max, s.hkv, s.batch), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(const msa_shape& s) {
  const Layout L = layout(s, MSA_KV_OUTER);
  const Geometry g = geometry(s, MSA_KV_OUTER);
  return L.total + align256((size_t)g.e_max * g.group * kD * 4);
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
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
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
  a.dq_part = reinterpret_cast<float*>(ws + L.total);
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
  if (g.nb_max > 0) {
    switch (g.group) {
      case 1: e = launch_kv_g<1>(s, g, a, st); break;
      case 2: e = launch_kv_g<2>(s, g, a, st); break;
      case 4: e = launch_kv_g<4>(s, g, a, st); break;
      case 8: e = launch_kv_g<8>(s, g, a, st); break;
      default: e = launch_kv_g<16>(s, g, a, st); break;
    }
    if (e != hipSuccess) return e;
  }
  const int64_t n = (int64_t)rows * 32;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const int32_t*>(ws + L.cmap), a.dq_part, dq, n, s.hq,
                     g.group, s.topk);
  return hipGetLastError();
}

}  // namespace msa
