// Per-Q-tile block selectors R1 and R4 ("Sparse Attention", Chapter 4: one or four
// representatives): each 128-query tile and each 128-key block is summarised, per head, by
// the mean of its tokens (R1) or the means of its four consecutive 32-token groups (R4); a
// block's score for a (tile, GQA group) is the largest dot product between a query
// representative of any head of the group and a key representative of the block; each tile
// and group keeps its top-K blocks, ordered by score descending then block ascending. The
// lists feed the per-Q-tile attention (list_q = 128).
//
// Three kernels:
//  - select_pool_kernel: the representatives (fp32), the token rows of a tile or block read
//    once with 16-byte loads;
//  - select_score_kernel: a workgroup scores a chunk of blocks for one (tile, group): the
//    chunk's key representatives go to LDS once, each thread keeps one query representative
//    in registers and forms its dot products with one key representative of each block, and
//    the maximum over a block's (head, representative) pairs is taken across lanes (and waves
//    when a block spans several) after all of them;
//  - select_topk_kernel: one wave per (tile, group) keeps a register top list per lane over
//    its share of the blocks, in ascending block order, and merges the 64 lists by a lane
//    tournament.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kSelectChunk = 16;   // blocks scored per workgroup

// Representatives of the units (tiles of queries or blocks of keys) of one sequence and
// head: out[(s * units_max + u) * heads + h][r][d] = mean of group r of unit u (0 for a group
// with no token; validity is recomputed from the lengths where scores are formed). Thread t
// sums dims 8 (t % 16) .. +7 of tokens 16 i + t / 16, i < 8: eight 16-byte loads issued before
// any is used; the 16 token lanes are then summed across the wave and the four waves.
template <int R>
__global__ __launch_bounds__(256) void select_pool_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ cu, float* __restrict__ out,
    int heads, int units_max, int total, int max_len) {
  constexpr int GS = kBlock / R;   // tokens per representative group
  __shared__ float red[4][R][kD];
  const int u = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 15, j = tid >> 4;
  const int t0 = min(max(cu[s], 0), total);
  const int t1 = min(max(cu[s + 1], t0), total);
  const int n = min(t1 - t0, max_len);
  const int base = u * kBlock;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = base + 16 * i + j;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (tok < n)
      v[i] = *reinterpret_cast<const u32x4*>(x + ((size_t)(t0 + tok) * heads + h) * kD + 8 * c);
  }
  float acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (16 * i) / GS;   // tokens 16 i .. 16 i + 15 lie in one group
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[r][2 * e] += bf16_bits_to_f32(v[i][e] & 0xFFFFu);
      acc[r][2 * e + 1] += bf16_bits_to_f32(v[i][e] >> 16);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[r][e] += shfl_xor_f(acc[r][e], 16);
      acc[r][e] += shfl_xor_f(acc[r][e], 32);
    }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][r][8 * c + e] = acc[r][e];
  }
  __syncthreads();
  float* o = out + (((size_t)s * units_max + u) * heads + h) * R * kD;
  for (int idx = tid; idx < R * kD; idx += 256) {
    const int r = idx / kD, d = idx % kD;
    const float sum = (red[0][r][d] + red[1][r][d]) + (red[2][r][d] + red[3][r][d]);
    const int cnt = min(max(n - base - r * GS, 0), GS);
    o[idx] = cnt > 0 ? sum / (float)cnt : 0.f;
  }
}

// Scores [(s * tiles_max + t) * hkv + g][nb_max] of one chunk of `cb` blocks; -inf where a
// block is past the sequence's end, invisible (causal) or has no comparable pair.
template <int R, int G>
__global__ __launch_bounds__(256) void select_score_kernel(
    const float* __restrict__ qrep, const float* __restrict__ krep,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    float* __restrict__ scores, int hkv, int tiles_max, int nb_max, int causal, int total_q,
    int total_k, int max_q, int max_k) {
  constexpr int GS = kBlock / R;
  constexpr int NQ = G * R;              // query representatives of a (tile, group)
  constexpr int P = NQ * R;              // (query rep, key rep) pairs of one block
  constexpr int BPP = 256 / P;           // blocks scored per pass
  constexpr int PW = P < 64 ? P : 64;    // lanes of a pair group inside one wave
  constexpr int NPASS = (kSelectChunk + BPP - 1) / BPP;
  __shared__ f32x4 kl[kSelectChunk * R * (kD / 4)];   // the chunk's key representatives
  __shared__ float red[4][NPASS];
  const int ts = blockIdx.x, g = blockIdx.y, chunk = blockIdx.z;
  const int s = ts / tiles_max, t = ts % tiles_max;
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  if (t * kBlock >= sq.nq) return;       // no such tile in this sequence
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = tid % P, bo = tid / P;
  const int qv = pair / R, kr = pair % R;
  const int h = g * G + qv / R, qi = qv % R;
  const bool q_ok = t * kBlock + qi * GS < sq.nq;
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  const int last = sq.nk - sq.nq + min(t * kBlock + kBlock - 1, sq.nq - 1);
  const int jvis = causal ? min(nb, floordiv(last, kBlock) + 1) : nb;
  const int b0 = chunk * kSelectChunk, b1 = min(b0 + kSelectChunk, nb);
  // the chunk's key representatives into LDS, 16 bytes per thread and load
  for (int i = tid; i < (b1 - b0) * R * (kD / 4); i += 256) {
    const int br = i / (kD / 4), q4 = i % (kD / 4);
    const int b = b0 + br / R, r = br % R;
    kl[i] = reinterpret_cast<const f32x4*>(krep + (((size_t)s * nb_max + b) * hkv + g) * R * kD +
                                           r * kD)[q4];
  }
  float qreg[kD];
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(
        qrep + (((size_t)ts * (hkv * G) + h) * R + qi) * kD);
#pragma unroll
    for (int i = 0; i < kD / 4; ++i) {
      const f32x4 v = src[i];
      qreg[4 * i] = v[0];
      qreg[4 * i + 1] = v[1];
      qreg[4 * i + 2] = v[2];
      qreg[4 * i + 3] = v[3];
    }
  }
  __syncthreads();
  float vals[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int b = b0 + p * BPP + bo;
    float v = -__builtin_inff();
    if (b < b1 && b < jvis && q_ok && b * kBlock + kr * GS < sq.nk) {
      const f32x4* src = kl + ((b - b0) * R + kr) * (kD / 4);
      // four partial sums (dims d mod 4) keep the FMA chains short
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int i = 0; i < kD / 4; ++i) {
        const f32x4 w = src[i];
        a0 = fmaf(qreg[4 * i], w[0], a0);
        a1 = fmaf(qreg[4 * i + 1], w[1], a1);
        a2 = fmaf(qreg[4 * i + 2], w[2], a2);
        a3 = fmaf(qreg[4 * i + 3], w[3], a3);
      }
      v = (a0 + a1) + (a2 + a3);
    }
    // maximum over the pairs of the block held by this wave's aligned lane group
#pragma unroll
    for (int off = 1; off < PW; off <<= 1) v = fmaxf(v, shfl_xor_f(v, off));
    vals[p] = v;
  }
  float* const srow = scores + (size_t)(ts * hkv + g) * nb_max;
  if constexpr (P > 64) {
    // a block's pairs span P / 64 waves
    if (lane == 0) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) red[wave][p] = vals[p];
    }
    __syncthreads();
    if (pair == 0) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        float v = vals[p];
#pragma unroll
        for (int w = 1; w < P / 64; ++w) v = fmaxf(v, red[wave + w][p]);
        const int b = b0 + p * BPP + bo;
        if (b < b1) srow[b] = v;
      }
    }
  } else {
    if (pair == 0) {
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const int b = b0 + p * BPP + bo;
        if (b < b1) srow[b] = vals[p];
      }
    }
  }
}

// Lists [(s * tiles_max + t) * hkv + g][topk] (and scores) from the block scores.
__global__ __launch_bounds__(64) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int32_t* __restrict__ lists, float* __restrict__ out_sc,
    int hkv, int tiles_max, int nb_max, int topk, int total_q, int total_k, int max_q,
    int max_k) {
  const int ts = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int s = ts / tiles_max, t = ts % tiles_max;
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  const size_t o = (size_t)(ts * hkv + g) * topk;
  const bool tile_ok = t * kBlock < sq.nq;
  const int nb = tile_ok ? (sq.nk + kBlock - 1) / kBlock : 0;
  const float* srow = scores + (size_t)(ts * hkv + g) * nb_max;
  TopList tl;
  tl.init();
  for (int b = lane; b < nb; b += 64) {
    const float v = srow[b];
    if (v > -__builtin_inff()) tl.insert(v, b);
  }
  for (int k = 0; k < topk; ++k) {
    float ws = tl.sc[0];
    int wi = tl.id[0];
    // wave arg-best: four levels on the DPP network, then lanes ^ 16 and ^ 32
    auto take = [&](float os, int oi) {
      if (beats(os, oi, ws, wi)) {
        ws = os;
        wi = oi;
      }
    };
    take(dpp_f<kDppXor1>(ws), dpp_i<kDppXor1>(wi));
    take(dpp_f<kDppXor2>(ws), dpp_i<kDppXor2>(wi));
    take(dpp_f<kDppHalfMirror>(ws), dpp_i<kDppHalfMirror>(wi));
    take(dpp_f<kDppMirror>(ws), dpp_i<kDppMirror>(wi));
    take(shfl_xor_f(ws, 16), shfl_xor_i(wi, 16));
    take(shfl_xor_f(ws, 32), shfl_xor_i(wi, 32));
    // the lane holding the winner drops it (each block sits in one lane's list)
    if (wi >= 0 && tl.id[0] == wi) {
#pragma unroll
      for (int q = 0; q + 1 < kMaxTopK; ++q) {
        tl.sc[q] = tl.sc[q + 1];
        tl.id[q] = tl.id[q + 1];
      }
      tl.sc[kMaxTopK - 1] = -__builtin_inff();
      tl.id[kMaxTopK - 1] = -1;
    }
    if (lane == 0) {
      lists[o + k] = wi;
      if (out_sc) out_sc[o + k] = wi >= 0 ? ws : -__builtin_inff();
    }
  }
}

template <int R, int G>
void launch_score_t(const msa_shape& s, const SelectGeometry& sg, const float* qrep,
                    const float* krep, const int32_t* cu_q, const int32_t* cu_k, float* scores,
                    hipStream_t st) {
  dim3 grid((unsigned)(s.batch * sg.tiles_max), s.hkv, (unsigned)sg.n_chunks);
  hipLaunchKernelGGL((select_score_kernel<R, G>), grid, dim3(256), 0, st, qrep, krep, cu_q,
                     cu_k, scores, s.hkv, (int)sg.tiles_max, (int)sg.nb_max, s.causal,
                     s.total_q, s.total_k, s.max_q, s.max_k);
}

template <int R>
void launch_score_r(const msa_shape& s, const SelectGeometry& sg, const float* qrep,
                    const float* krep, const int32_t* cu_q, const int32_t* cu_k, float* scores,
                    hipStream_t st) {
  switch (s.hq / s.hkv) {
    case 1: launch_score_t<R, 1>(s, sg, qrep, krep, cu_q, cu_k, scores, st); break;
    case 2: launch_score_t<R, 2>(s, sg, qrep, krep, cu_q, cu_k, scores, st); break;
    case 4: launch_score_t<R, 4>(s, sg, qrep, krep, cu_q, cu_k, scores, st); break;
    case 8: launch_score_t<R, 8>(s, sg, qrep, krep, cu_q, cu_k, scores, st); break;
    default: launch_score_t<R, 16>(s, sg, qrep, krep, cu_q, cu_k, scores, st); break;
  }
}

}  // namespace

SelectGeometry select_geometry(const msa_shape& s, int reps) {
  SelectGeometry sg{};
  sg.reps = reps;
  sg.tiles_max = cdiv(s.max_q, kBlock);
  sg.nb_max = cdiv(s.max_k, kBlock);
  // chunks of 16 blocks: (tiles x groups x chunks) workgroups fill the chip at the pages'
  // shapes (4096 queries, 16K keys, one group: 64 x 8 = 512)
  sg.chunk = kSelectChunk;
  sg.n_chunks = std::max<int64_t>(1, cdiv(sg.nb_max, sg.chunk));
  const size_t qrep = (size_t)s.batch * sg.tiles_max * s.hq * reps * kD * 4;
  const size_t krep = (size_t)s.batch * sg.nb_max * s.hkv * reps * kD * 4;
  const size_t sc = (size_t)s.batch * sg.tiles_max * s.hkv * sg.nb_max * 4;
  sg.off_qrep = 0;
  sg.off_krep = align256(qrep);
  sg.off_scores = sg.off_krep + align256(krep);
  sg.total = sg.off_scores + align256(sc);
  return sg;
}

hipError_t launch_select_tiles(const msa_shape& s, int reps, const void* q, const void* k,
                               const int32_t* cu_q, const int32_t* cu_k, int32_t* lists,
                               float* scores, char* ws, hipStream_t st) {
  const SelectGeometry sg = select_geometry(s, reps);
  if (sg.tiles_max == 0) return hipSuccess;
  float* const qrep = reinterpret_cast<float*>(ws + sg.off_qrep);
  float* const krep = reinterpret_cast<float*>(ws + sg.off_krep);
  float* const sc = reinterpret_cast<float*>(ws + sg.off_scores);
  const dim3 gq((unsigned)sg.tiles_max, s.hq, s.batch);   // 256 threads per (unit, head)
  if (reps == 1)
    hipLaunchKernelGGL(select_pool_kernel<1>, gq, dim3(256), 0, st, (const uint16_t*)q, cu_q,
                       qrep, s.hq, (int)sg.tiles_max, s.total_q, s.max_q);
  else
    hipLaunchKernelGGL(select_pool_kernel<4>, gq, dim3(256), 0, st, (const uint16_t*)q, cu_q,
                       qrep, s.hq, (int)sg.tiles_max, s.total_q, s.max_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sg.nb_max > 0) {
    const dim3 gk((unsigned)sg.nb_max, s.hkv, s.batch);
    if (reps == 1)
      hipLaunchKernelGGL(select_pool_kernel<1>, gk, dim3(256), 0, st, (const uint16_t*)k, cu_k,
                         krep, s.hkv, (int)sg.nb_max, s.total_k, s.max_k);
    else
      hipLaunchKernelGGL(select_pool_kernel<4>, gk, dim3(256), 0, st, (const uint16_t*)k, cu_k,
                         krep, s.hkv, (int)sg.nb_max, s.total_k, s.max_k);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (reps == 1)
      launch_score_r<1>(s, sg, qrep, krep, cu_q, cu_k, sc, st);
    else
      launch_score_r<4>(s, sg, qrep, krep, cu_q, cu_k, sc, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 gt((unsigned)(s.batch * sg.tiles_max), s.hkv);
  hipLaunchKernelGGL(select_topk_kernel, gt, dim3(64), 0, st, sc, cu_q, cu_k, lists, scores,
                     s.hkv, (int)sg.tiles_max, (int)sg.nb_max, s.topk, s.total_q, s.total_k,
                     s.max_q, s.max_k);
  return hipGetLastError();
}

}  // namespace msa
