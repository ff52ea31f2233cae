// Log-sum-exp combine of per-slot partial outputs.
//
// "Sparse Attention" (Chapter 5, partial outputs and combine): combine weights each partial
// by its LSE relative to the others; "Kernel optimization for MiniMax M3 on NVIDIA
// Blackwell" (section 2): the combine kernel is bandwidth-bound and gathers the partials
// through the (query, kv head, slot) -> location map.
//
// A thread owns 8 output dims (16 bytes) of one (query, head): it reads the slot LSEs and
// weight sums, then issues all of its slot loads before accumulating, so each wave keeps 16
// independent 1 KiB gathers in flight. Partials are read in their 8-row group layout. A partial is stored unnormalised (its output times its
// weight sum l), so slot k enters with coefficient exp(lse_k - m) / l_k.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

template <int G>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ cmap,
                                                      const int32_t* __restrict__ counters,
                                                      const float* __restrict__ part_lse,
                                                      const float* __restrict__ part_l,
                                                      const uint16_t* __restrict__ part_o,
                                                      uint16_t* __restrict__ o,
                                                      float* __restrict__ lse, int total_q,
                                                      int hkv, int slots) {
  constexpr int TPB = G * 16;               // threads per (query, group) box
  constexpr int BOXES = 256 / TPB;
  const int tid = threadIdx.x;
  // Boxes from the last query backwards (1% faster than the forward order at the M3 shape;
  // the partials are written with streaming stores, which a probe shows do not stay in the
  // last-level cache, so little of them is still cached either way).
  const int64_t n_boxes = (int64_t)total_q * hkv;
  const int64_t idx = (int64_t)blockIdx.x * BOXES + tid / TPB;
  if (idx >= n_boxes) return;
  const int box = (int)(n_boxes - 1 - idx);
  // the thread's (head, 16-byte chunk): with G >= 8 an entry's G rows are whole 8-row groups
  // of the partial layout and thread j of the box reads its bytes 16 j .. 16 j + 15 (each
  // wave 1 KiB of consecutive bytes; its output stores fill 8 whole rows' halves)
  const int j = tid % TPB;
  const int g = G >= 8 ? 8 * (j >> 7) + (j & 7) : j % G;
  const int c = G >= 8 ? (j >> 3) & 15 : j / G;
  const int t = box / hkv, h = box % hkv;
  const int n_ent = counters[0];
  const int hq = hkv * G;
  const int32_t* cm = cmap + ((size_t)t * hkv + h) * slots;

  // Slot indices first; then the LSE loads and the 16-byte partial loads of every valid
  // slot are all issued before any of them is used.
  int es[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    int e = -1;
    if (k < slots) e = cm[k];
    es[k] = (e >= n_ent) ? -1 : e;
  }
  float ls[kMaxTopK], lw[kMaxTopK];
  u32x4 vals[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    u32x4 v = {0u, 0u, 0u, 0u};
    float l = -__builtin_inff(), w = 1.f;
    if (es[k] >= 0) {
      l = part_lse[(size_t)es[k] * G + g];
      w = part_l[(size_t)es[k] * G + g];
      // streaming load: each partial is read exactly once
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          reinterpret_cast<const char*>(part_o) + part_chunk_offset((size_t)es[k] * G + g, c)));
    }
    ls[k] = l;
    lw[k] = w;
    vals[k] = v;
  }
  float m = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) m = fmaxf(m, ls[k]);
  uint16_t* orow = o + ((size_t)t * hq + h * G + g) * kD + 8 * c;
  if (!(m > -__builtin_inff())) {
    *reinterpret_cast<u32x4*>(orow) = u32x4{0u, 0u, 0u, 0u};
    if (lse && c == 0) lse[(size_t)t * hq + h * G + g] = -__builtin_inff();
    return;
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float wsum = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    const float w = __builtin_amdgcn_exp2f((ls[k] - m) * 1.4426950408889634f);  // 0 for -inf
    wsum += w;
    const float cw = w > 0.f ? w * __builtin_amdgcn_rcpf(lw[k]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(cw, bf16_bits_to_f32(vals[k][i] & 0xFFFFu), acc[2 * i]);
      acc[2 * i + 1] = fmaf(cw, bf16_bits_to_f32(vals[k][i] >> 16), acc[2 * i + 1]);
    }
  }
  const float inv = 1.f / wsum;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(orow) = out;
  if (lse && c == 0) lse[(size_t)t * hq + h * G + g] = m + logf(wsum);
}

}  // namespace

hipError_t launch_combine(const msa_shape& s, const Geometry& g, const Layout& L,
                          const char* ws, void* o, float* lse, hipStream_t st) {
  if (s.total_q == 0) return hipSuccess;
  const int tpb = g.group * 16;
  const int boxes = 256 / tpb;
  const int64_t n_boxes = (int64_t)s.total_q * s.hkv;
  dim3 grid((unsigned)((n_boxes + boxes - 1) / boxes));
  const int32_t* cmap = reinterpret_cast<const int32_t*>(ws + L.cmap);
  const int32_t* cnt = reinterpret_cast<const int32_t*>(ws + L.counters);
  const float* pl = reinterpret_cast<const float*>(ws + L.part_lse);
  const float* pw = reinterpret_cast<const float*>(ws + L.part_l);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(ws + L.part_o);
  uint16_t* oo = reinterpret_cast<uint16_t*>(o);
  switch (g.group) {
    case 1: hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, st, cmap, cnt, pl, pw, po, oo, lse, s.total_q, s.hkv, L.slots); break;
    case 2: hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, st, cmap, cnt, pl, pw, po, oo, lse, s.total_q, s.hkv, L.slots); break;
    case 4: hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, st, cmap, cnt, pl, pw, po, oo, lse, s.total_q, s.hkv, L.slots); break;
    case 8: hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, st, cmap, cnt, pl, pw, po, oo, lse, s.total_q, s.hkv, L.slots); break;
    default: hipLaunchKernelGGL(combine_kernel<16>, grid, dim3(256), 0, st, cmap, cnt, pl, pw, po, oo, lse, s.total_q, s.hkv, L.slots); break;
  }
  return hipGetLastError();
}

}  // namespace msa
