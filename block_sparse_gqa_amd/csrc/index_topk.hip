// Index branch: max-pooled proxy block scores and streaming top-K with the local block forced.
//
// "Flash-MSA: accelerating million-token training" (proxy forward): as each tile of proxy
// scores is produced, the causal max of each 128-key chunk is inserted into a per-row top-K
// kept in registers, and the query's local block gets an infinite score. "Kernel
// optimization for MiniMax M3 on NVIDIA Blackwell" (summary): one selection per GQA group.
//
// Two kernels compute the same result:
//  - index_tile_kernel (prefill): a workgroup owns 256 queries of one group and streams the
//    proxy key blocks through LDS; S^T = K_idx Q_idx^T on bf16 MFMA puts one query per lane
//    column, so a block max is an in-register max plus one cross-lane exchange.
//  - index_split_kernel + index_merge_kernel (few queries, e.g. decode): the key range is
//    cut into chunks of blocks scored by separate workgroups (a bandwidth-bound scan of the
//    proxy keys); their top-K lists are merged by (score desc, block asc).
// Blocks are always visited in ascending order and inserted only on a strictly greater
// score, so equal scores keep the lower block index first.
#include <algorithm>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kIndexTileQ = 256;   // queries per workgroup of the tile kernel (64 per wave)

// Proxy precisions: bf16, OCP fp8 e4m3 with per-tensor descales, OCP MXFP4 (E2M1 codes, two
// per byte with the even element in the low nibble, one E8M0 scale byte per 32 elements).
enum : int { kPrBf16 = 0, kPrFp8 = 1, kPrFp4 = 2 };
// bytes of one proxy row of DP elements
template <int PR>
constexpr int proxy_row_bytes(int dp) {
  return PR == kPrBf16 ? 2 * dp : (PR == kPrFp8 ? dp : dp / 2);
}
// E8M0 code -> its power of two (code 0: 2^-127, a subnormal)
__device__ __forceinline__ float e8m0_to_f32(unsigned e) {
  return e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// Blocks the tile kernel scores for query tile `tile` of a sequence: those before the local
// block of the tile's last query (causal), or all of them.
__device__ __forceinline__ int tile_blocks(const Seq& sq, int tile, int causal) {
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  if (!causal) return nb;
  const int il_last = min(tile * kIndexTileQ + kIndexTileQ - 1, sq.nq - 1);
  return max(0, min(floordiv(sq.nk - sq.nq + il_last, kBlock), nb));
}
constexpr float kPosInf = __builtin_inff();

// `scale` turns raw proxy dot products into scores (fp8 proxies: the two descales).
__device__ __forceinline__ void write_list(int32_t* out_idx, float* out_sc, int topk,
                                           bool has_local, int local, const float* sc,
                                           const int* id, float scale) {
  int base = 0;
  if (has_local) {
    out_idx[0] = local;
    if (out_sc) out_sc[0] = kPosInf;
    base = 1;
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (base + k < topk) {
      out_idx[base + k] = id[k];
      if (out_sc) out_sc[base + k] = id[k] >= 0 ? sc[k] * scale : kNegInf;
    }
  }
}

// ------------------------------------------------------------------------ tile kernel
// s_waitcnt vmcnt(n) for the direct-to-LDS loads of the block ring (not tracked by the
// compiler's own waits).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 MFMA on OCP e4m3 operands (scales 2^0): lane l supplies row l % 32 of A (column
// l % 32 of B) at contraction indices 32 (l / 32) .. +31; the result has the layout of the
// bf16 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 0, 0, 0, 127, 0, 127);
}
// The same MFMA on MXFP4 operands: lane l supplies 32 E2M1 codes (16 bytes; the instruction
// reads four registers) of row l % 32 at contraction indices 32 (l / 32) .. +31, which is one
// scale group, and that group's E8M0 scale byte (sa for A, sb for B).
__device__ __forceinline__ f32x16 mfma_f4(const i32x8& a, const i32x8& b, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 4, 4, 0, sa, 0, sb);
}
__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A workgroup scores one 256-query tile of one group against every block it can see,
// heavy (late, causal) tiles first. (Splitting long tiles' key ranges over several
// workgroups, with a merge of the partial lists, measured slower at 32K and 128K keys.)
// FP8: e4m3 proxies ("Sparse Attention", Chapter 4: a scorer on low-precision index vectors),
// one 8-bit MFMA per 32 x 32 score tile over the whole proxy dim (dp = 32 fills the upper
// half of the 64-long contraction with zeros); scores are the raw dot products times the two
// descales, applied where they are written (a positive factor does not change the order).
// FP4: MXFP4 proxies ("Sparse Attention", Chapter 4: the scorer on 4-bit index vectors), one
// scaled 4-bit MFMA per score tile, each lane's scale byte beside its 32 codes; the key
// blocks' scale bytes are read into registers one pair of blocks ahead.
template <int DP, int PR>
__global__ __launch_bounds__(256) void index_tile_kernel(
    const void* __restrict__ q_idx_, const void* __restrict__ k_idx_,
    const uint8_t* __restrict__ q_sc, const uint8_t* __restrict__ k_sc,
    const float* __restrict__ descale_idx, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_score, int hkv, int topk, int causal, int total_q, int total_k,
    int max_q, int max_k, int one_round) {
  constexpr bool FP8 = PR == kPrFp8, FP4 = PR == kPrFp4;
  constexpr int RB = proxy_row_bytes<PR>(DP);   // bytes per proxy row
  constexpr int CH = RB / 16;      // 16-byte chunks per proxy key row
  constexpr int STEPS = DP / 16;   // bf16 MFMA k-steps over the proxy dim
  constexpr int NCK = 128 * CH;    // chunks per key block
  constexpr int PER_T = NCK >= 256 ? NCK / 256 : 1;   // direct-to-LDS loads per thread per block
  constexpr int NSC = DP / 32;     // FP4: scale bytes per proxy row
  const char* const q_idx = reinterpret_cast<const char*>(q_idx_);
  const char* const k_idx = reinterpret_cast<const char*>(k_idx_);
  constexpr int NBUF = 4;          // ring of key blocks: two pairs
  __shared__ u32x4 kl[NBUF][128 * CH];

  const int s = blockIdx.z, h = blockIdx.y;
  // Causal tiles grow with their position; heavy tiles go first. When the whole grid runs in
  // one round (two workgroups per compute unit), the second half of the (sequence, group)
  // pairs takes its tiles light first instead: the workgroups that share a compute unit (the
  // dispatcher fills every unit once, then again in the same order) then pair a heavy tile
  // with a light one instead of two of the same size.
  const bool light_first =
      one_round && (int)(s * gridDim.y + h) >= (int)(gridDim.y * gridDim.z) / 2;
  const int tile = light_first ? (int)blockIdx.x : (int)(gridDim.x - 1 - blockIdx.x);
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  if (tile * kIndexTileQ >= sq.nq) return;

  // A wave scores 64 queries as two 32-query halves (one per MFMA B operand), so each K
  // operand read from LDS feeds two MFMAs. Lane (col, hf) keeps the top list of query
  // col of half hf.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int q_wave = tile * kIndexTileQ + wave * 64;
  const int il = q_wave + hf * 32 + col;
  const bool qvalid = il < sq.nq;
  const int pos = sq.nk - sq.nq + il;
  const int c = floordiv(pos, kBlock);

  const int jbeg = 0, jend = tile_blocks(sq, tile, causal);

  bf16x8 bq[2][STEPS];
  i32x8 bq8[2];
  int qsc[2] = {127, 127};   // FP4: this lane's query scale byte per half
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int iq = q_wave + qh * 32 + col;
    const bool ok = iq < sq.nq;
    const size_t qr = (size_t)(sq.q0 + (ok ? iq : 0)) * hkv + h;
    const char* qrow = q_idx + qr * RB;
    if constexpr (FP4) {
      // bytes 16 hf .. 16 hf + 15 of the row: scale group hf (dp = 32: half 1 holds zeros)
      u32x4 w = {0u, 0u, 0u, 0u};
      const u32x4 z = {0u, 0u, 0u, 0u};
      if (ok && (DP == 64 || hf == 0)) {
        w = *reinterpret_cast<const u32x4*>(qrow + 16 * hf);
        qsc[qh] = q_sc[qr * NSC + hf];
      }
      bq8[qh] = cat8(w, z);
    } else if constexpr (FP8) {
      // bytes 32 hf .. 32 hf + 31 of the row (dp = 32: the lanes of half 1 hold zeros)
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (ok && (DP == 64 || hf == 0)) {
        lo = *reinterpret_cast<const u32x4*>(qrow + 32 * hf);
        hi = *reinterpret_cast<const u32x4*>(qrow + 32 * hf + 16);
      }
      bq8[qh] = cat8(lo, hi);
    } else {
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = *reinterpret_cast<const u32x4*>(qrow + 32 * st + 16 * hf);
        bq[qh][st] = as_bf16x8(v);
      }
    }
  }

  TopList tl;
  tl.init();

  // Block j into ring slot j % NBUF. Slot i of the buffer (16 bytes) holds chunk
  // (i % CH) ^ f(row) of key row i / CH, f(row) = (row / 2) % CH: lane l of each load fetches
  // the chunk that belongs in the slot it writes, so a load covers whole rows. Rows past the
  // end of the sequence repeat its last key, which belongs to the same (last) block: the
  // repeats cannot change the block's maximum, so no masking is needed.
  // Thread t covers rows t / CH + (256 / CH) p, p < PER_T, all at chunk slot t % CH; the
  // swizzle term (row / 2) % CH is the same for all of them.
  const unsigned row0 = (unsigned)tid / CH;
  const unsigned cc0 = ((unsigned)tid % CH) ^ ((row0 >> 1) & (CH - 1));
  const size_t krow = (size_t)hkv * RB;                 // bytes between consecutive keys
  const char* const kh = k_idx + (size_t)h * RB + cc0 * 16;
  auto dma_block = [&](int j) {
    if (NCK < 256 && wave >= NCK / 64) return;   // fewer chunks than threads (fp4, dp = 32)
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const unsigned row = row0 + (256 / CH) * p;
      const unsigned u = min(j * kBlock + (int)row, sq.nk - 1);
      __builtin_amdgcn_global_load_lds(
          kh + (size_t)(sq.k0 + u) * krow,
          (__attribute__((address_space(3))) void*)(&kl[j % NBUF][p * 256 + wave * 64]), 16, 0,
          0);
    }
  };

  // FP4: the scale bytes this lane's K operands need in block j (key rows kt * 32 + col,
  // scale group hf; the last key repeats past the end, like the rows)
  int ksc[2][4], ksc_next[2][4];
  auto load_ksc = [&](int j, int (&dst)[4]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int u = min(j * kBlock + kt * 32 + col, sq.nk - 1);
      dst[kt] = (DP == 64 || hf == 0) ? (int)k_sc[((size_t)(sq.k0 + u) * hkv + h) * NSC + hf]
                                      : 127;
    }
  };

  // Blocks go through the ring in pairs: pair (jp, jp + 1) is scored while the next pair
  // loads into the two slots the previous pair has just left, so one wait and one barrier
  // serve two blocks.
  for (int j = jbeg; j < min(jend, jbeg + 2); ++j) dma_block(j);
  // (constant register indices and clamped block numbers: a load into a runtime-indexed
  // register array would be waited for at once, together with the block loads before it)
  if constexpr (FP4) {
    if (jend > jbeg) {
      load_ksc(jbeg, ksc[0]);
      load_ksc(min(jbeg + 1, jend - 1), ksc[1]);
    }
  }
  for (int jp = jbeg; jp < jend; jp += 2) {
    wait_vm<0>();      // this thread's parts of the pair have landed (nothing else in flight)
    __syncthreads();   // every thread's parts are in LDS; the previous pair's slots are free
    for (int j = jp + 2; j < min(jp + 4, jend); ++j) dma_block(j);
    if constexpr (FP4) {
      load_ksc(min(jp + 2, jend - 1), ksc_next[0]);
      load_ksc(min(jp + 3, jend - 1), ksc_next[1]);
    }
    for (int j = jp; j < min(jp + 2, jend); ++j) {
    const int buf = j % NBUF;

    f32x16 acc[2][4];
    if constexpr (FP4) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int row = kt * 32 + col;
        const int sw = (row >> 1) & (CH - 1);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 w = kl[buf][row * CH + ((DP == 64 ? hf : 0) ^ sw)];
        const i32x8 ka = (DP == 64 || hf == 0) ? cat8(w, z) : cat8(z, z);
        const int sa = (j - jp) ? ksc[1][kt] : ksc[0][kt];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) acc[qh][kt] = mfma_f4(ka, bq8[qh], sa, qsc[qh]);
      }
    } else if constexpr (FP8) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int row = kt * 32 + col;
        const int sw = (row >> 1) & (CH - 1);
        const int c0 = DP == 64 ? 2 * hf : 0;
        const u32x4 lo = kl[buf][row * CH + (c0 ^ sw)];
        const u32x4 hi = kl[buf][row * CH + ((c0 + 1) ^ sw)];
        const u32x4 z = {0u, 0u, 0u, 0u};
        const i32x8 ka = (DP == 64 || hf == 0) ? cat8(lo, hi) : cat8(z, z);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) acc[qh][kt] = mfma_f8(ka, bq8[qh]);
      }
    } else {
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        bf16x8 ka[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int row = kt * 32 + col;
          const int cc = 2 * st + hf;
          ka[kt] = as_bf16x8(kl[buf][row * CH + (cc ^ ((row >> 1) & (CH - 1)))]);
        }
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            acc[qh][kt] = mfma32(ka[kt], bq[qh][st], st == 0 ? f32x16{} : acc[qh][kt]);
      }
    }
    float mq[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      float m4[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        m4[kt] = acc[qh][kt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m4[kt] = fmaxf(m4[kt], acc[qh][kt][r]);
      }
      mq[qh] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
      mq[qh] = fmaxf(mq[qh], shfl_xor_f(mq[qh], 32));   // both lanes of the column
    }
    const float mx = hf ? mq[1] : mq[0];
    // insertion only where the block beats the current last entry (wave-uniform skip)
    const bool ins = qvalid && (causal ? (j < c) : (j != c)) && mx > tl.sc[kMaxTopK - 1];
    if (__any(ins)) {
      if (ins) tl.insert(mx, j);
    }
    }
    if constexpr (FP4) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) ksc[b][kt] = ksc_next[b][kt];
    }
  }

  if (qvalid) {
    const size_t o = ((size_t)(sq.q0 + il) * hkv + h) * topk;
    const float scale = FP8 ? descale_idx[0] * descale_idx[1] : 1.f;
    write_list(topk_idx + o, topk_score ? topk_score + o : nullptr, topk, pos >= 0, c, tl.sc,
               tl.id, scale);
  }
}

// ------------------------------------------------------------------------ split kernels
// Grid: x = key chunk, y = sequence * max_q + query. One workgroup scores the chunk's blocks
// for every group: with hkv >= 4 wave w takes groups w, w+4, ..., each over all of the chunk's
// blocks; with hkv < 4 the 4/hkv waves of a group take its blocks in turn. The waves thus read
// the groups' interleaved proxy-key rows of the same keys together, i.e. one contiguous span
// of memory (the scan is bound by HBM bandwidth). Dot products on the VALUs; the chunk's list
// of each group (merged in LDS over the waves sharing the group) goes to the workspace.
template <int DP, int PR>
__global__ __launch_bounds__(256) void index_split_kernel(
    const void* __restrict__ q_idx_, const void* __restrict__ k_idx_,
    const uint8_t* __restrict__ q_sc, const uint8_t* __restrict__ k_sc,
    const float* __restrict__ descale_idx, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, float* __restrict__ part_sc, int32_t* __restrict__ part_id,
    int hkv, int max_q, int causal, int n_chunks, int chunk_blocks, int total_q, int total_k,
    int max_k) {
  constexpr bool FP8 = PR == kPrFp8, FP4 = PR == kPrFp4;
  constexpr int RB = proxy_row_bytes<PR>(DP);   // bytes per proxy row
  constexpr int VPL = FP4 ? 32 : (FP8 ? 16 : 8);  // proxy elements per lane (16 bytes)
  constexpr int LPK = RB / 16;     // lanes per key row
  constexpr int NSC = DP / 32;     // FP4: scale bytes per row (lane dc holds scale group dc)
  constexpr int KPI = 64 / LPK;    // keys per wave instruction
  const char* const q_idx = reinterpret_cast<const char*>(q_idx_);
  const char* const k_idx = reinterpret_cast<const char*>(k_idx_);
  // partial scores leave the kernel scaled (fp8: the two descales); the merge compares them
  const float scale = FP8 ? descale_idx[0] * descale_idx[1] : 1.f;
  __shared__ float lsc[4][kMaxTopK];
  __shared__ int lid[4][kMaxTopK];

  const int chunk = blockIdx.x;
  const int s = blockIdx.y / max_q, il = blockIdx.y % max_q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  const bool qvalid = il < sq.nq;
  const int pos = sq.nk - sq.nq + il;
  const int c = floordiv(pos, kBlock);
  const int nb = (sq.nk + kBlock - 1) / kBlock;
  const int jend = qvalid ? (causal ? min(max(c, 0), nb) : nb) : 0;
  const int j0 = chunk * chunk_blocks;
  const int j1 = min(j0 + chunk_blocks, jend);
  const int wph = hkv >= 4 ? 1 : 4 / hkv;   // waves per group
  const int kk = lane / LPK, dc = lane % LPK;

  // this wave's best blocks of group h over blocks j0 + sub, j0 + sub + wph, ...
  // the 16 bytes of a lane as VPL floats (bf16, e4m3 codes or E2M1 codes, unscaled)
  auto unpack = [](const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (FP4) {
        // byte b of the word: elements 2b (low nibble) and 2b + 1
        const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.f, 0);
        const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.f, 1);
        const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.f, 2);
        const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.f, 3);
        f[8 * i] = v0[0];
        f[8 * i + 1] = v0[1];
        f[8 * i + 2] = v1[0];
        f[8 * i + 3] = v1[1];
        f[8 * i + 4] = v2[0];
        f[8 * i + 5] = v2[1];
        f[8 * i + 6] = v3[0];
        f[8 * i + 7] = v3[1];
      } else if constexpr (FP8) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        f[4 * i] = lo[0];
        f[4 * i + 1] = lo[1];
        f[4 * i + 2] = hi[0];
        f[4 * i + 3] = hi[1];
      } else {
        f[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  };
  auto scan = [&](int h, int sub, TopList& tl) {
    float qv[VPL];
    float qs = 1.f;   // FP4: the query's scale of group dc
    {
      u32x4 w = {0u, 0u, 0u, 0u};
      const size_t qr = (size_t)(sq.q0 + il) * hkv + h;
      if (qvalid) {
        w = *reinterpret_cast<const u32x4*>(q_idx + qr * RB + dc * 16);
        if constexpr (FP4) qs = e8m0_to_f32(q_sc[qr * NSC + dc]);
      }
      unpack(w, qv);
    }
    tl.init();
    for (int j = j0 + sub; j < j1; j += wph) {
      if (!causal && j == c) continue;
      float mx = kNegInf;
      constexpr int IT = kBlock / KPI;
      u32x4 kvv[IT];
      unsigned ksv[IT];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int u = j * kBlock + it * KPI + kk;
        u32x4 w = {0u, 0u, 0u, 0u};
        ksv[it] = 127u;
        if (u < sq.nk) {
          const size_t kr = (size_t)(sq.k0 + u) * hkv + h;
          w = *reinterpret_cast<const u32x4*>(k_idx + kr * RB + dc * 16);
          if constexpr (FP4) ksv[it] = k_sc[kr * NSC + dc];
        }
        kvv[it] = w;
      }
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float kv[VPL];
        unpack(kvv[it], kv);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) dot = fmaf(qv[i], kv[i], dot);
        // FP4: the group's products are exact and so is their sum (multiples of 1/4 below
        // 2^11); the two scales are powers of two, so only the sum over groups rounds
        if constexpr (FP4) dot = dot * qs * e8m0_to_f32(ksv[it]);
        dot = group_sum<LPK>(dot);
        const int u = j * kBlock + it * KPI + kk;
        if (u >= sq.nk) dot = kNegInf;
        mx = fmaxf(mx, dot);
      }
      mx = wave_max_from<LPK>(mx);
      if (mx > tl.sc[kMaxTopK - 1]) tl.insert(mx, j);   // (wave-uniform: skips no-op insertions)
    }
  };
  auto out_base = [&](int h) {
    return ((((size_t)s * max_q + il) * hkv + h) * n_chunks + chunk) * kMaxTopK;
  };

  if (wph == 1) {
    // a wave per group: its list is the chunk's list (empty slots are -inf / -1)
    for (int h = wave; h < hkv; h += 4) {
      TopList tl;
      scan(h, 0, tl);
      if (lane == 0) {
        const size_t base = out_base(h);
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
          part_sc[base + k] = tl.sc[k] * scale;
          part_id[base + k] = tl.id[k];
        }
      }
    }
    return;
  }
  const int h = wave % hkv, sub = wave / hkv;
  TopList tl;
  scan(h, sub, tl);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      lsc[wave][k] = tl.sc[k];
      lid[wave][k] = tl.id[k];
    }
  }
  __syncthreads();
  if (sub == 0) {
    // the group's wph * 16 candidates, one per lane (lists of waves h, h + hkv, ...): rank =
    // number of candidates that beat it
    const int n_cand = wph * kMaxTopK;
    const int lw = h + (lane >> 4) * hkv;
    const float sc = lane < n_cand ? lsc[lw][lane & 15] : kNegInf;
    const int id = lane < n_cand ? lid[lw][lane & 15] : -1;
    int rank = 0, n_real = 0;
    for (int o = 0; o < n_cand; ++o) {
      const int ow = h + (o >> 4) * hkv;
      const float os = lsc[ow][o & 15];
      const int oi = lid[ow][o & 15];
      rank += beats(os, oi, sc, id) ? 1 : 0;
      n_real += oi >= 0 ? 1 : 0;
    }
    const size_t base = out_base(h);
    if (id >= 0 && rank < kMaxTopK) {
      part_sc[base + rank] = sc * scale;
      part_id[base + rank] = id;
    }
    // slots past the number of real candidates are empty
    if (lane < kMaxTopK && lane >= n_real) {
      part_sc[base + lane] = kNegInf;
      part_id[base + lane] = -1;
    }
  }
}

// One wave per (sequence, query, group): every chunk list is read once into registers (lane
// l merges lists l, l + 64, ... into one list), then K rounds of a tournament over the lanes'
// list heads, the winning lane shifting its list.
__global__ __launch_bounds__(64) void index_merge_kernel(
    const float* __restrict__ part_sc, const int32_t* __restrict__ part_id,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_score, int hkv, int max_q,
    int topk, int n_chunks, int total_q, int total_k, int max_k) {
  const int h = blockIdx.y;
  const int s = blockIdx.x / max_q, il = blockIdx.x % max_q;
  const int lane = threadIdx.x;
  const Seq sq = load_seq_clamped(cu_q, cu_k, s, total_q, total_k, max_q, max_k);
  if (il >= sq.nq) return;
  const int pos = sq.nk - sq.nq + il;
  const int c = floordiv(pos, kBlock);
  const bool has_local = pos >= 0;
  const size_t base = (((size_t)s * max_q + il) * hkv + h) * n_chunks;

  // this lane's lists, in chunk order (ties then keep the lower block, as in one scan)
  TopList tl;
  tl.init();
  for (int li = lane; li < n_chunks; li += 64) {
    const u32x4* ps = reinterpret_cast<const u32x4*>(part_sc + (base + li) * kMaxTopK);
    const u32x4* pi = reinterpret_cast<const u32x4*>(part_id + (base + li) * kMaxTopK);
    u32x4 vs[4], vi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vs[q] = ps[q];
      vi[q] = pi[q];
    }
    if (li == lane) {
      // the first list is already sorted: take it as it is
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        tl.sc[k] = __uint_as_float(vs[k >> 2][k & 3]);
        tl.id[k] = (int)vi[k >> 2][k & 3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        const int id = (int)vi[k >> 2][k & 3];
        if (id >= 0) tl.insert(__uint_as_float(vs[k >> 2][k & 3]), id);
      }
    }
  }

  float out_sc[kMaxTopK];
  int out_id[kMaxTopK];
  const int need = topk - (has_local ? 1 : 0);
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    float ws = tl.sc[0];
    int wi = tl.id[0];
    // wave arg-best: four levels on the DPP network, then lanes ^ 16 and ^ 32
    auto take = [&](float os, int oi) {
      if (beats(os, oi, ws, wi)) { ws = os; wi = oi; }
    };
    take(dpp_f<kDppXor1>(ws), dpp_i<kDppXor1>(wi));
    take(dpp_f<kDppXor2>(ws), dpp_i<kDppXor2>(wi));
    take(dpp_f<kDppHalfMirror>(ws), dpp_i<kDppHalfMirror>(wi));
    take(dpp_f<kDppMirror>(ws), dpp_i<kDppMirror>(wi));
    take(shfl_xor_f(ws, 16), shfl_xor_i(wi, 16));
    take(shfl_xor_f(ws, 32), shfl_xor_i(wi, 32));
    out_sc[k] = ws;
    out_id[k] = wi;
    // the lane holding the winner drops it (block ids are unique across lists)
    if (wi >= 0 && tl.id[0] == wi) {
#pragma unroll
      for (int q = 0; q + 1 < kMaxTopK; ++q) {
        tl.sc[q] = tl.sc[q + 1];
        tl.id[q] = tl.id[q + 1];
      }
      tl.sc[kMaxTopK - 1] = kNegInf;
      tl.id[kMaxTopK - 1] = -1;
    }
    if (k + 1 >= need) break;
  }
  if (lane == 0) {
    const size_t o = ((size_t)(sq.q0 + il) * hkv + h) * topk;
    // (the chunk lists' scores are already scaled)
    write_list(topk_idx + o, topk_score ? topk_score + o : nullptr, topk, has_local, c, out_sc,
               out_id, 1.f);
  }
}

}  // namespace

// Key chunks of the split kernel (short-query calls) per (sequence, query, group).
static int64_t index_chunks(const msa_shape& s) {
  const int64_t nb_max = (s.max_k + s.block - 1) / s.block;
  const int cb = split_index_chunk(nb_max);
  return std::max<int64_t>(1, (nb_max + cb - 1) / cb);
}

size_t index_workspace_bytes(const msa_shape& s) {
  if (s.max_q > kSplitIndexMaxQ) return 0;
  const int64_t n = (int64_t)s.batch * s.max_q * s.hkv * index_chunks(s) * kMaxTopK;
  return (size_t)n * 8 + 256;
}

static hipError_t launch_index_merge(const msa_shape& s, const float* part_sc,
                                     const int32_t* part_id, int n_chunks, const int32_t* cu_q,
                                     const int32_t* cu_k, int32_t* topk_idx, float* topk_score,
                                     hipStream_t st) {
  dim3 grid2(s.batch * s.max_q, s.hkv);
  hipLaunchKernelGGL(index_merge_kernel, grid2, dim3(64), 0, st, part_sc, part_id, cu_q, cu_k,
                     topk_idx, topk_score, s.hkv, s.max_q, s.topk, n_chunks, s.total_q,
                     s.total_k, s.max_k);
  return hipGetLastError();
}

template <int DP, int PR>
static void launch_tile_t(const msa_shape& s, dim3 grid, const IndexProxies& px,
                          const int32_t* cu_q, const int32_t* cu_k, int32_t* topk_idx,
                          float* topk_score, int one_round, hipStream_t st) {
  hipLaunchKernelGGL((index_tile_kernel<DP, PR>), grid, dim3(256), 0, st, px.q_idx, px.k_idx,
                     px.q_scale, px.k_scale, px.descale, cu_q, cu_k, topk_idx, topk_score, s.hkv,
                     s.topk, s.causal, s.total_q, s.total_k, s.max_q, s.max_k, one_round);
}

template <int PR>
static void launch_tile_p(const msa_shape& s, dim3 grid, const IndexProxies& px,
                          const int32_t* cu_q, const int32_t* cu_k, int32_t* topk_idx,
                          float* topk_score, int one_round, hipStream_t st) {
  if (s.dp == 64)
    launch_tile_t<64, PR>(s, grid, px, cu_q, cu_k, topk_idx, topk_score, one_round, st);
  else
    launch_tile_t<32, PR>(s, grid, px, cu_q, cu_k, topk_idx, topk_score, one_round, st);
}

hipError_t launch_index_tile(const msa_shape& s, const IndexProxies& px, const int32_t* cu_q,
                             const int32_t* cu_k, int32_t* topk_idx, float* topk_score,
                             hipStream_t st) {
  const int tiles = (s.max_q + kIndexTileQ - 1) / kIndexTileQ;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, s.hkv, s.batch);
  const int one_round = (int64_t)tiles * s.hkv * s.batch <= 2 * (int64_t)device_cu_count();
  switch (px.prec) {
    case kIdxFp8:
      launch_tile_p<kPrFp8>(s, grid, px, cu_q, cu_k, topk_idx, topk_score, one_round, st);
      break;
    case kIdxMxfp4:
      launch_tile_p<kPrFp4>(s, grid, px, cu_q, cu_k, topk_idx, topk_score, one_round, st);
      break;
    default:
      launch_tile_p<kPrBf16>(s, grid, px, cu_q, cu_k, topk_idx, topk_score, one_round, st);
  }
  return hipGetLastError();
}

template <int DP, int PR>
static void launch_split_t(const msa_shape& s, dim3 grid, const IndexProxies& px,
                           const int32_t* cu_q, const int32_t* cu_k, float* part_sc,
                           int32_t* part_id, int n_chunks, int cb, hipStream_t st) {
  hipLaunchKernelGGL((index_split_kernel<DP, PR>), grid, dim3(256), 0, st, px.q_idx, px.k_idx,
                     px.q_scale, px.k_scale, px.descale, cu_q, cu_k, part_sc, part_id, s.hkv,
                     s.max_q, s.causal, n_chunks, cb, s.total_q, s.total_k, s.max_k);
}

template <int PR>
static void launch_split_p(const msa_shape& s, dim3 grid, const IndexProxies& px,
                           const int32_t* cu_q, const int32_t* cu_k, float* part_sc,
                           int32_t* part_id, int n_chunks, int cb, hipStream_t st) {
  if (s.dp == 64)
    launch_split_t<64, PR>(s, grid, px, cu_q, cu_k, part_sc, part_id, n_chunks, cb, st);
  else
    launch_split_t<32, PR>(s, grid, px, cu_q, cu_k, part_sc, part_id, n_chunks, cb, st);
}

hipError_t launch_index_split(const msa_shape& s, const IndexProxies& px, const int32_t* cu_q,
                              const int32_t* cu_k, int32_t* topk_idx, float* topk_score,
                              void* ws, hipStream_t st) {
  if (s.max_q == 0) return hipSuccess;
  const int64_t nb_max = (s.max_k + s.block - 1) / s.block;
  const int cb = split_index_chunk(nb_max);
  const int n_chunks = (int)((nb_max + cb - 1) / cb);
  const int64_t n = (int64_t)s.batch * s.max_q * s.hkv * n_chunks * kMaxTopK;
  float* part_sc = reinterpret_cast<float*>(ws);
  int32_t* part_id = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + n * 4);
  if (n_chunks > 0) {
    dim3 grid(n_chunks, s.batch * s.max_q);
    switch (px.prec) {
      case kIdxFp8:
        launch_split_p<kPrFp8>(s, grid, px, cu_q, cu_k, part_sc, part_id, n_chunks, cb, st);
        break;
      case kIdxMxfp4:
        launch_split_p<kPrFp4>(s, grid, px, cu_q, cu_k, part_sc, part_id, n_chunks, cb, st);
        break;
      default:
        launch_split_p<kPrBf16>(s, grid, px, cu_q, cu_k, part_sc, part_id, n_chunks, cb, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_index_merge(s, part_sc, part_id, n_chunks, cu_q, cu_k, topk_idx, topk_score, st);
}

}  // namespace msa
