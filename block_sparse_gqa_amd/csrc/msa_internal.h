// Host-side internals of libmsa: workspace plan and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Threshold below which the index branch splits the key range across workgroups instead of
// tiling queries (decode and other short-query calls).
constexpr int kSplitIndexMaxQ = 16;
// Blocks of keys scored by one workgroup of the split index kernel: 8 up to 1024 blocks (128
// chunks; twice the workgroups of 16-block chunks: fp8 and 4-bit decode scans 8% faster, bf16
// the same), 32 beyond (the merge reads at most 512 chunk lists).
constexpr int kSplitIndexChunk = 32;
inline int split_index_chunk(int64_t nb_max) { return nb_max <= 1024 ? 8 : kSplitIndexChunk; }
// Queries per inverted-index bitmap word.
constexpr int kWordQ = 64;
// Queries per range of the entry order (s, group, range, block, query). The attention
// kernels hand each (s, group, range) phase to one XCD, whose workgroups split the phase's
// tiles. Longer ranges hold more queries per bucket (fuller tiles, fewer K/V loads) but more
// Q rows per phase: bf16 takes up to 1024 queries (16 heads x 256 B x 1024 = 4 MiB, one XCD's
// L2: at the M3 shape 3.21 ms with 512, 3.10 with 1024, 3.11 with 2048), fp8 up to 2048 (the
// same 4 MiB of e4m3 rows: at 128K tokens 10.23 / 9.80 / 9.91 ms with 1024 / 2048 / 4096);
// either as long as the schedule keeps at least 128 phases (16 per XCD) to spread, and never
// below 512.
constexpr int kRangeQMin = 512;
constexpr int kRangeQBf16Max = 1024;
constexpr int kRangeQFp8Max = 2048;
constexpr int64_t kMinPhases = 128;
inline int range_q(const msa_shape& s) {
  int r = s.dtype == MSA_FP8_E4M3 ? kRangeQFp8Max : kRangeQBf16Max;
  while (r > kRangeQMin &&
         (int64_t)s.batch * s.hkv * ((s.max_q + (int64_t)r - 1) / r) < kMinPhases)
    r /= 2;
  return r;
}
// Elements per workgroup in the scan kernels.
constexpr int kScanTile = 4096;

struct Geometry {
  int64_t nb_max;        // ceil(max_k / block)
  int64_t w_max;         // ceil(max_q / 64): bitmap words per (sequence, group, block)
  int64_t wr;            // bitmap words per bucket (power of two, <= range_q / 64)
  int64_t n_r;           // query ranges per sequence: ceil(w_max / wr)
  int64_t n_buckets;     // batch * hkv * n_r * nb_max
  int64_t n_phase;       // batch * hkv * n_r: (sequence, group, range) phases
  int64_t n_tiles_max;   // bound on attention tiles (entries split per bucket into tiles)
  int64_t n_words;       // n_buckets * w_max
  int64_t e_max;         // total_q * hkv * topk (upper bound on entries)
  int64_t n_scan_blocks; // ceil(n_words / kScanTile)
  int64_t n_lists;       // rows of topk_idx: total_q, or batch * tiles_max for tile lists
  int64_t tiles_max;     // ceil(max_q / list_q)
  int group;             // hq / hkv
  int splits;            // Q-outer: splits of each list (1 = output written directly)
  int64_t index_chunks;  // split index kernel: key chunks per sequence
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Offsets (bytes) of each region of the caller's workspace.
struct Layout {
  size_t counters;      // int32[64]: [0] = number of entries
  size_t masks;         // uint64 [n_words]
  size_t offsets;       // int32  [n_words + 1]
  size_t scan_sums;     // int32  [n_scan_blocks + 1]
  size_t entry_q;       // int32  [e_max]
  size_t entry_bucket;  // int32  [e_max]
  size_t cmap;          // int32  [total_q * hkv * slots]
  size_t tile_off;      // int32  [n_buckets]: first tile of each bucket, phase-relative
  size_t phase_base;    // int32  [2 * (n_phase + 1)]: first tile record of each phase,
                        //   then the tile count of each phase
  size_t tiles;         // int2   [n_tiles_max]: (first entry, block << 8 | entries - 1)
  size_t v_wide;        // bf16   [total_k * hkv * d]: fp8 V widened (KV-outer fp8 only)
  size_t part_lse;      // float  [e_max * group]
  size_t part_l;        // float  [e_max * group]: weight sums (partials are unnormalised)
  size_t part_o;        // bf16   [e_max * group * d]
  size_t total;
  int slots;            // combine slots per (query, group): topk or splits
};

Geometry geometry(const msa_shape& s, msa_mode mode);
Layout layout(const msa_shape& s, msa_mode mode);
size_t index_workspace_bytes(const msa_shape& s);

// ----- launchers (return hipSuccess or the launch error)
// Proxies of the index branch: bf16; fp8 e4m3 with device descales descale[0] (q_idx),
// descale[1] (k_idx); MXFP4 codes (two per byte, even element in the low nibble) with one
// E8M0 scale byte per 32 elements in q_scale / k_scale ([token, group, dp / 32]).
enum IndexPrec : int { kIdxBf16 = 0, kIdxFp8 = 1, kIdxMxfp4 = 2 };
struct IndexProxies {
  IndexPrec prec;
  const void* q_idx;
  const void* k_idx;
  const uint8_t* q_scale;
  const uint8_t* k_scale;
  const float* descale;
};
hipError_t launch_index_tile(const msa_shape& s, const IndexProxies& px, const int32_t* cu_q,
                             const int32_t* cu_k, int32_t* topk_idx, float* topk_score,
                             hipStream_t st);
hipError_t launch_index_split(const msa_shape& s, const IndexProxies& px, const int32_t* cu_q,
                              const int32_t* cu_k, int32_t* topk_idx, float* topk_score,
                              void* ws, hipStream_t st);

// Per-Q-tile selectors R1 / R4: the workspace regions (query and key representatives, fp32;
// block scores) and the block chunks of the scoring kernel.
struct SelectGeometry {
  int reps;
  int chunk;             // blocks scored per workgroup
  int64_t tiles_max, nb_max, n_chunks;
  size_t off_qrep, off_krep, off_scores, total;
};
SelectGeometry select_geometry(const msa_shape& s, int reps);
hipError_t launch_select_tiles(const msa_shape& s, int reps, const void* q, const void* k,
                               const int32_t* cu_q, const int32_t* cu_k, int32_t* lists,
                               float* scores, char* ws, hipStream_t st);

hipError_t launch_plan(const msa_shape& s, const Geometry& g, const Layout& L,
                       const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k,
                       char* ws, hipStream_t st);
hipError_t launch_attn_kv(const msa_shape& s, const Geometry& g, const Layout& L,
                          const void* q, const void* k, const void* v, const float* descale,
                          float scale, const int32_t* cu_q, const int32_t* cu_k, char* ws,
                          hipStream_t st);
hipError_t launch_attn_q(const msa_shape& s, const Geometry& g, const Layout& L,
                         const void* q, const void* k, const void* v, const float* descale,
                         float scale, const int32_t* lists, const int32_t* cu_q,
                         const int32_t* cu_k, char* ws, void* o, float* lse, hipStream_t st);
// Read-bandwidth probe: kProbeGrid workgroups of 256 threads, 4 KiB per workgroup and pass.
constexpr int kProbeGrid = 1024;
hipError_t launch_probe_read(const void* buf, size_t working_set, size_t total, float* sink,
                             hipStream_t st);
hipError_t launch_combine(const msa_shape& s, const Geometry& g, const Layout& L,
                          const char* ws, void* o, float* lse, hipStream_t st);
// Main-branch backward: workspace = the KV-outer plan, bf16 dQ partials [E, group, d], the
// chunk map and fp32 dK / dV partials of chunks of split columns.
size_t bwd_workspace_bytes(const msa_shape& s);
bool bwd_fits(const msa_shape& s);
// Proxy backward: workspace = the KV-outer plan, fp32 dq_idx partials [E, dp], the chunk map,
// fp32 dk_idx partials of chunks of split columns and the proxy LSE [total_q, hkv].
size_t proxy_bwd_workspace_bytes(const msa_shape& s);
hipError_t launch_proxy_bwd(const msa_shape& s, const void* q, const void* k, const void* q_idx,
                            const void* k_idx, const float* lse, float scale, float proxy_scale,
                            const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k,
                            char* ws, float* dq_idx, float* dk_idx, float* lse_proxy,
                            hipStream_t st);   // chunk and column counts within 32-bit indexing
hipError_t launch_bwd(const msa_shape& s, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dout, float scale,
                      const int32_t* lists, const int32_t* cu_q, const int32_t* cu_k, char* ws,
                      float* dq, float* dk, float* dv, hipStream_t st);

int device_cu_count();
int device_xcd_count();

}  // namespace msa
