// C ABI of libmsa: argument checks, workspace plan, schedule choice, kernel dispatch.
// Host code only; every check runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

thread_local std::string g_last_error;

constexpr int64_t kInt32Max = 2147483647LL;

msa_status check_shape(const msa_shape* s) {
  if (!s) return MSA_ERR_NULL;
  if (s->dtype != MSA_BF16 && s->dtype != MSA_FP8_E4M3) return MSA_ERR_DTYPE;
  if (s->batch < 1 || s->batch > 65535) return MSA_ERR_SHAPE;
  if (s->total_q < 0 || s->total_k < 0 || s->max_q < 0 || s->max_k < 0) return MSA_ERR_SHAPE;
  if (s->hq < 1 || s->hkv < 1 || s->hq % s->hkv != 0 || s->hq > 65535) return MSA_ERR_SHAPE;
  const int g = s->hq / s->hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return MSA_ERR_SHAPE;
  if (s->d != kD || s->block != kBlock) return MSA_ERR_SHAPE;
  if (s->topk < 1 || s->topk > kMaxTopK) return MSA_ERR_SHAPE;
  if (s->causal != 0 && s->causal != 1) return MSA_ERR_SHAPE;
  if (s->list_q != 1 && s->list_q != 128) return MSA_ERR_SHAPE;
  if (s->max_q > s->total_q || s->max_k > s->total_k) return MSA_ERR_SHAPE;
  // 32-bit indexing of entries, partial rows and token rows
  if ((int64_t)s->total_q * s->hkv * s->topk * g > kInt32Max) return MSA_ERR_SHAPE;
  if ((int64_t)s->total_q * s->hq > kInt32Max || (int64_t)s->total_k * s->hkv > kInt32Max)
    return MSA_ERR_SHAPE;
  return MSA_OK;
}

// Splits of each per-query list for the Q-outer kernel: the smallest power of two giving about
// one workgroup per compute unit of a 256-CU part for bf16 (its kernel holds two blocks in
// LDS, one workgroup per CU) and two for fp8 (one block, two workgroups per CU), so that each
// workgroup streams its blocks back to back. Shape-only, so the workspace size depends on the
// shape alone.
int choose_splits(const msa_shape& s) {
  const int64_t target = s.dtype == MSA_BF16 ? 256 : 512;
  int ns = 1;
  while (ns * 2 <= s.topk && (int64_t)s.total_q * s.hkv * ns < target) ns *= 2;
  return ns;
}

// Effective cache-to-HBM bandwidth ratio of the Q-outer re-reads on MI355X, measured: the
// probe reads 5.91 TB/s from HBM, 7.80 TB/s from the last-level cache (working sets of 64 to
// 192 MiB; ratio 1.32) and 29.6 TB/s from the XCDs' L2 (16 MiB); timing both schedules over
// block reuse nsb/N = 64 .. 1/32 (2048 queries, Hq = 64, Hkv = 4, top-16, bf16) puts the
// crossover at nsb/N = 19.2, which the byte model below gives for a ratio of 2.32 (part of the
// re-reads hit the L2). The last-level cache ratio alone would give 40.
constexpr double kCacheToHbmRatio = 2.32;

double crossover_x(const msa_shape& s, double bw_hbm, double bw_cache) {
  const double e = s.dtype == MSA_FP8_E4M3 ? 1.0 : 2.0;
  const double hq = s.hq, hkv = s.hkv, d = s.d, k = s.topk, bk = s.block;
  const double kv_per_n = hq * d * e + hq * k * (2.0 * 2.0 * d + 2.0 * 4.0) + hq * d * 2.0;
  const double q_per_n = hkv * k * 2.0 * bk * d * e + hq * d * (e + 2.0);
  const double beta = bw_cache / bw_hbm;
  return (q_per_n / beta - kv_per_n) / (2.0 * bk * d * e);
}

msa_mode resolve(const msa_shape& s, msa_mode mode) {
  if (mode != MSA_AUTO) return mode;
  if (s.list_q > 1) return MSA_Q_OUTER;
  const int64_t nb_max = cdiv(s.max_k, s.block);
  const double nsb = (double)std::min<int64_t>((int64_t)s.batch * s.hkv * nb_max,
                                               (int64_t)s.total_q * s.hkv * s.topk);
  if (s.total_q == 0) return MSA_KV_OUTER;
  const double x = crossover_x(s, 1.0, kCacheToHbmRatio);
  return (nsb / s.total_q < x) ? MSA_KV_OUTER : MSA_Q_OUTER;
}

msa_status check_mode(const msa_shape& s, msa_mode mode, msa_mode* out) {
  if (mode != MSA_AUTO && mode != MSA_KV_OUTER && mode != MSA_Q_OUTER) return MSA_ERR_MODE;
  const msa_mode m = resolve(s, mode);
  if (m == MSA_KV_OUTER) {
    const int64_t nb_max = cdiv(s.max_k, s.block);
    if (nb_max > 8192) return MSA_ERR_SHAPE;           // LDS bitmap tile of the plan
    const Geometry g = geometry(s, m);
    if (g.n_words + 1 > kInt32Max) return MSA_ERR_SHAPE;   // 32-bit scan
    if (g.n_tiles_max > kInt32Max) return MSA_ERR_SHAPE;
  }
  *out = m;
  return MSA_OK;
}

void fail_launch(hipError_t e) { g_last_error = hipGetErrorString(e); }

}  // namespace

Geometry geometry(const msa_shape& s, msa_mode mode) {
  Geometry g{};
  g.group = s.hq / s.hkv;
  g.nb_max = cdiv(s.max_k, s.block);
  g.tiles_max = cdiv(s.max_q, s.list_q);
  g.n_lists = s.list_q == 1 ? s.total_q : (int64_t)s.batch * g.tiles_max;
  g.splits = 1;
  if (mode == MSA_KV_OUTER) {
    g.w_max = cdiv(s.max_q, kWordQ);
    g.wr = 1;
    while (g.wr < g.w_max && g.wr < range_q(s) / kWordQ) g.wr *= 2;
    g.n_r = cdiv(g.w_max, g.wr);
    g.n_phase = (int64_t)s.batch * s.hkv * g.n_r;
    g.n_buckets = g.n_phase * g.nb_max;
    g.n_words = g.n_buckets * g.wr;
    g.e_max = (int64_t)s.total_q * s.hkv * s.topk;
    // a bucket of c entries makes ceil(c / (256 / group)) tiles
    g.n_tiles_max = std::min(g.e_max, g.e_max / (256 / g.group) + g.n_buckets) + 1;
    g.n_scan_blocks = cdiv(g.n_words, kScanTile);
  } else {
    g.splits = s.list_q == 1 ? choose_splits(s) : 1;
    g.e_max = g.splits > 1 ? (int64_t)s.total_q * s.hkv * g.splits : 0;
  }
  return g;
}

Layout layout(const msa_shape& s, msa_mode mode) {
  const Geometry g = geometry(s, mode);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.counters = take(64 * 4);
  if (mode == MSA_KV_OUTER) {
    L.slots = s.topk;
    L.masks = take((size_t)g.n_words * 8);
    L.offsets = take((size_t)(g.n_words + 1) * 4);
    L.scan_sums = take((size_t)(g.n_scan_blocks + 1) * 4);
    L.entry_q = take((size_t)g.e_max * 4);
    L.entry_bucket = take((size_t)g.e_max * 4);
    L.cmap = take((size_t)s.total_q * s.hkv * s.topk * 4);
    L.tile_off = take((size_t)g.n_buckets * 4);
    L.phase_base = take((size_t)(g.n_phase + 1) * 8);
    L.tiles = take((size_t)g.n_tiles_max * 8);
    // bf16 V^T of every (group, key block) (e4m3 V widened exactly), blocks numbered per
    // sequence from its first key: ceil(total_k / 128) + batch per group
    L.v_wide = take((size_t)s.hkv * (cdiv(s.total_k, s.block) + s.batch) * s.block * s.d * 2);
  } else {
    L.slots = g.splits;
    L.masks = L.offsets = L.scan_sums = L.entry_q = L.entry_bucket = off;
    L.tile_off = L.phase_base = L.tiles = L.v_wide = off;
    L.cmap = take(g.splits > 1 ? (size_t)s.total_q * s.hkv * g.splits * 4 : 0);
  }
  L.part_lse = take((size_t)g.e_max * g.group * 4);
  L.part_l = take((size_t)g.e_max * g.group * 4);
  // partial rows in groups of 8 (see the partial layout of the kernels)
  L.part_o = take((size_t)((g.e_max * g.group + 7) / 8 * 8) * s.d * 2);
  L.total = off;
  return L;
}

// XCDs of the device (chiplets with their own L2). The tiled attention kernel gives each XCD
// its own query ranges; workgroup i is taken to run on XCD i % n (round-robin dispatch).
// Only locality depends on this, never the result.
int device_xcd_count() {
  const int cu = device_cu_count();
  return cu % 8 == 0 ? 8 : 1;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace msa


// Scratch of the allocation-free main-branch call: one array per device, kept until the
// process ends. In host code `scratch` names a host-side stand-in, not device memory: every
// host use goes through the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace msa {
namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (nullptr and an error text on failure).
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_error = e != hipSuccess ? hipGetErrorString(e) : "device index out of range";
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = e != hipSuccess ? hipGetErrorString(e) : "scratch has no device address";
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

const char* msa_status_string(msa_status st) {
  switch (st) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "null pointer argument";
    case MSA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case MSA_ERR_DTYPE: return "unknown dtype";
    case MSA_ERR_WORKSPACE: return "workspace missing or too small";
    case MSA_ERR_MODE: return "mode not allowed";
    case MSA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

msa_status msa_resolve_mode(const msa_shape* shape, msa_mode mode, msa_mode* chosen) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!chosen) return MSA_ERR_NULL;
  return check_mode(*shape, mode, chosen);
}

msa_status msa_crossover(const msa_shape* shape, double bw_hbm, double bw_cache, double* x) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!x) return MSA_ERR_NULL;
  if (!(bw_hbm > 0)) return MSA_ERR_SHAPE;
  if (bw_cache <= 0) bw_cache = kCacheToHbmRatio * bw_hbm;
  *x = crossover_x(*shape, bw_hbm, bw_cache);
  return MSA_OK;
}

msa_status msa_workspace_layout_of(const msa_shape* shape, msa_mode mode,
                                   msa_workspace_layout* out) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!out) return MSA_ERR_NULL;
  msa_mode m;
  st = check_mode(*shape, mode, &m);
  if (st != MSA_OK) return st;
  const Layout L = layout(*shape, m);
  const Geometry g = geometry(*shape, m);
  out->counters = L.counters;
  out->masks = L.masks;
  out->offsets = L.offsets;
  out->scan_sums = L.scan_sums;
  out->entry_q = L.entry_q;
  out->entry_bucket = L.entry_bucket;
  out->cmap = L.cmap;
  out->part_lse = L.part_lse;
  out->part_l = L.part_l;
  out->part_o = L.part_o;
  out->v_wide = L.v_wide;
  out->total = L.total;
  out->slots = L.slots;
  out->n_words = (int32_t)g.n_words;
  out->w_max = (int32_t)g.w_max;
  out->words_per_bucket = (int32_t)g.wr;
  out->n_ranges = (int32_t)g.n_r;
  out->nb_max = (int32_t)g.nb_max;
  return MSA_OK;
}

msa_status msa_workspace_size(const msa_shape* shape, msa_mode mode, size_t* bytes) {
  if (!bytes) return MSA_ERR_NULL;
  msa_workspace_layout L;
  msa_status st = msa_workspace_layout_of(shape, mode, &L);
  if (st != MSA_OK) return st;
  *bytes = L.total;
  return MSA_OK;
}

msa_status msa_index_workspace_size(const msa_shape* shape, size_t* bytes) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_NULL;
  *bytes = index_workspace_bytes(*shape);
  return MSA_OK;
}

static msa_status index_topk(const msa_shape* shape, const IndexProxies& px,
                             const int32_t* cu_q, const int32_t* cu_k, int32_t* topk_idx,
                             float* topk_score, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.list_q != 1 || (s.dp != 32 && s.dp != 64)) return MSA_ERR_SHAPE;
  if ((int64_t)s.total_q * s.hkv * s.dp > kInt32Max * 2LL) return MSA_ERR_SHAPE;
  if (!cu_q || !cu_k || !topk_idx) return MSA_ERR_NULL;
  if (s.total_q > 0 && !px.q_idx) return MSA_ERR_NULL;
  if (s.total_k > 0 && !px.k_idx) return MSA_ERR_NULL;
  if (px.prec == kIdxFp8 && !px.descale) return MSA_ERR_NULL;
  if (px.prec == kIdxMxfp4 && ((s.total_q > 0 && !px.q_scale) || (s.total_k > 0 && !px.k_scale)))
    return MSA_ERR_NULL;
  hipError_t e;
  if (s.max_q <= kSplitIndexMaxQ) {
    // key chunks merged by one wave per (query, group): at most 512 per query
    if (cdiv(cdiv(s.max_k, s.block), kSplitIndexChunk) > 512) return MSA_ERR_SHAPE;
    if ((int64_t)s.batch * s.max_q > 65535) return MSA_ERR_SHAPE;      // grid y of the split kernel
    const size_t need = index_workspace_bytes(s);
    if (!workspace || ws_bytes < need) return MSA_ERR_WORKSPACE;
    e = launch_index_split(s, px, cu_q, cu_k, topk_idx, topk_score, workspace, stream);
  } else {
    e = launch_index_tile(s, px, cu_q, cu_k, topk_idx, topk_score, stream);
  }
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_index_topk(const msa_shape* shape, const void* q_idx, const void* k_idx,
                          const int32_t* cu_q, const int32_t* cu_k, int32_t* topk_idx,
                          float* topk_score, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  const IndexProxies px{kIdxBf16, q_idx, k_idx, nullptr, nullptr, nullptr};
  return index_topk(shape, px, cu_q, cu_k, topk_idx, topk_score, workspace, ws_bytes, stream);
}

msa_status msa_index_topk_fp8(const msa_shape* shape, const void* q_idx, const void* k_idx,
                              const float* descale_idx, const int32_t* cu_q, const int32_t* cu_k,
                              int32_t* topk_idx, float* topk_score, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  const IndexProxies px{kIdxFp8, q_idx, k_idx, nullptr, nullptr, descale_idx};
  return index_topk(shape, px, cu_q, cu_k, topk_idx, topk_score, workspace, ws_bytes, stream);
}

msa_status msa_index_topk_mxfp4(const msa_shape* shape, const void* q_idx,
                                const uint8_t* q_scale, const void* k_idx,
                                const uint8_t* k_scale, const int32_t* cu_q, const int32_t* cu_k,
                                int32_t* topk_idx, float* topk_score, void* workspace,
                                size_t ws_bytes, hipStream_t stream) {
  const IndexProxies px{kIdxMxfp4, q_idx, k_idx, q_scale, k_scale, nullptr};
  return index_topk(shape, px, cu_q, cu_k, topk_idx, topk_score, workspace, ws_bytes, stream);
}

msa_status msa_select_workspace_size(const msa_shape* shape, int reps, size_t* bytes) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_NULL;
  if (reps != 1 && reps != 4) return MSA_ERR_SHAPE;
  *bytes = select_geometry(*shape, reps).total;
  return MSA_OK;
}

msa_status msa_select_tiles(const msa_shape* shape, int reps, const void* q, const void* k,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t* lists,
                            float* scores, void* workspace, size_t ws_bytes,
                            hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (s.list_q != kBlock || (reps != 1 && reps != 4)) return MSA_ERR_SHAPE;
  const SelectGeometry sg = select_geometry(s, reps);
  if (sg.n_chunks > 65535 || (int64_t)s.batch * sg.tiles_max > kInt32Max) return MSA_ERR_SHAPE;
  if (!cu_q || !cu_k || !lists) return MSA_ERR_NULL;
  if ((s.total_q > 0 && !q) || (s.total_k > 0 && !k)) return MSA_ERR_NULL;
  if (!workspace || ws_bytes < sg.total) return MSA_ERR_WORKSPACE;
  const hipError_t e = launch_select_tiles(s, reps, q, k, cu_q, cu_k, lists, scores,
                                           static_cast<char*>(workspace), stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_bwd_workspace_size(const msa_shape* shape, size_t* bytes) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_NULL;
  if (shape->dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(*shape)) return MSA_ERR_SHAPE;
  *bytes = bwd_workspace_bytes(*shape);
  return MSA_OK;
}

msa_status msa_sparse_attn_bwd(const msa_shape* shape, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dout,
                               float softmax_scale, const int32_t* topk_idx,
                               const int32_t* cu_q, const int32_t* cu_k, void* workspace,
                               size_t ws_bytes, float* dq, float* dk, float* dv,
                               hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(s)) return MSA_ERR_SHAPE;
  if (!topk_idx || !cu_q || !cu_k) return MSA_ERR_NULL;
  if (s.total_q > 0 && (!q || !o || !lse || !dout || !dq)) return MSA_ERR_NULL;
  if (s.total_k > 0 && (!k || !v || !dk || !dv)) return MSA_ERR_NULL;
  if (!workspace || ws_bytes < bwd_workspace_bytes(s)) return MSA_ERR_WORKSPACE;
  const hipError_t e = launch_bwd(s, q, k, v, o, lse, dout, softmax_scale, topk_idx, cu_q, cu_k,
                                  static_cast<char*>(workspace), dq, dk, dv, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_train_bwd_workspace_size(const msa_shape* shape, size_t* bytes) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_NULL;
  if (shape->dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(*shape) || (shape->dp != 32 && shape->dp != 64)) return MSA_ERR_SHAPE;
  *bytes = std::max(bwd_workspace_bytes(*shape), proxy_bwd_workspace_bytes(*shape));
  return MSA_OK;
}

msa_status msa_train_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout, float softmax_scale,
                         const void* q_idx, const void* k_idx, float proxy_scale,
                         const int32_t* topk_idx, const int32_t* cu_q, const int32_t* cu_k,
                         void* workspace, size_t ws_bytes, float* dq, float* dk, float* dv,
                         float* dq_idx, float* dk_idx, float* lse_proxy, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(s) || (s.dp != 32 && s.dp != 64)) return MSA_ERR_SHAPE;
  if (!topk_idx || !cu_q || !cu_k) return MSA_ERR_NULL;
  if (s.total_q > 0 && (!q || !o || !lse || !dout || !dq || !q_idx || !dq_idx))
    return MSA_ERR_NULL;
  if (s.total_k > 0 && (!k || !v || !dk || !dv || !k_idx || !dk_idx)) return MSA_ERR_NULL;
  if (!workspace || ws_bytes < std::max(bwd_workspace_bytes(s), proxy_bwd_workspace_bytes(s)))
    return MSA_ERR_WORKSPACE;
  // the two passes one after the other on the caller's stream, sharing the workspace
  hipError_t e = launch_bwd(s, q, k, v, o, lse, dout, softmax_scale, topk_idx, cu_q, cu_k,
                            static_cast<char*>(workspace), dq, dk, dv, stream);
  if (e == hipSuccess)
    e = launch_proxy_bwd(s, q, k, q_idx, k_idx, lse, softmax_scale, proxy_scale, topk_idx, cu_q,
                         cu_k, static_cast<char*>(workspace), dq_idx, dk_idx, lse_proxy, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_proxy_bwd_workspace_size(const msa_shape* shape, size_t* bytes) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  if (!bytes) return MSA_ERR_NULL;
  if (shape->dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(*shape) || (shape->dp != 32 && shape->dp != 64)) return MSA_ERR_SHAPE;
  *bytes = proxy_bwd_workspace_bytes(*shape);
  return MSA_OK;
}

msa_status msa_proxy_attn_bwd(const msa_shape* shape, const void* q, const void* k,
                              const void* q_idx, const void* k_idx, const float* lse,
                              float softmax_scale, float proxy_scale, const int32_t* topk_idx,
                              const int32_t* cu_q, const int32_t* cu_k, void* workspace,
                              size_t ws_bytes, float* dq_idx, float* dk_idx, float* lse_proxy,
                              hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (s.dtype != MSA_BF16) return MSA_ERR_DTYPE;
  if (!bwd_fits(s) || (s.dp != 32 && s.dp != 64)) return MSA_ERR_SHAPE;
  if (!topk_idx || !cu_q || !cu_k) return MSA_ERR_NULL;
  if (s.total_q > 0 && (!q || !q_idx || !lse || !dq_idx)) return MSA_ERR_NULL;
  if (s.total_k > 0 && (!k || !k_idx || !dk_idx)) return MSA_ERR_NULL;
  if (!workspace || ws_bytes < proxy_bwd_workspace_bytes(s)) return MSA_ERR_WORKSPACE;
  const hipError_t e = launch_proxy_bwd(s, q, k, q_idx, k_idx, lse, softmax_scale, proxy_scale,
                                        topk_idx, cu_q, cu_k, static_cast<char*>(workspace),
                                        dq_idx, dk_idx, lse_proxy, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

static msa_status prep(const msa_shape* shape, msa_mode mode, const void* workspace,
                       size_t ws_bytes, msa_mode* m, Geometry* g, Layout* L) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  st = check_mode(*shape, mode, m);
  if (st != MSA_OK) return st;
  *g = geometry(*shape, *m);
  *L = layout(*shape, *m);
  if (!workspace || ws_bytes < L->total) return MSA_ERR_WORKSPACE;
  return MSA_OK;
}

msa_status msa_plan(const msa_shape* shape, const int32_t* topk_idx, const int32_t* cu_q,
                    const int32_t* cu_k, void* workspace, size_t ws_bytes, hipStream_t stream) {
  msa_mode m;
  Geometry g;
  Layout L;
  msa_status st = prep(shape, MSA_KV_OUTER, workspace, ws_bytes, &m, &g, &L);
  if (st != MSA_OK) return st;
  if (!topk_idx || !cu_q || !cu_k) return MSA_ERR_NULL;
  hipError_t e = launch_plan(*shape, g, L, topk_idx, cu_q, cu_k, (char*)workspace, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_attn_main(const msa_shape* shape, const void* q, const void* k, const void* v,
                         const float* descale_qkv, float softmax_scale, const int32_t* cu_q,
                         const int32_t* cu_k, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  msa_mode m;
  Geometry g;
  Layout L;
  msa_status st = prep(shape, MSA_KV_OUTER, workspace, ws_bytes, &m, &g, &L);
  if (st != MSA_OK) return st;
  if (!cu_q || !cu_k) return MSA_ERR_NULL;
  if ((shape->total_q > 0 && !q) || (shape->total_k > 0 && (!k || !v))) return MSA_ERR_NULL;
  if (shape->dtype == MSA_FP8_E4M3 && !descale_qkv) return MSA_ERR_NULL;
  hipError_t e = launch_attn_kv(*shape, g, L, q, k, v, descale_qkv, softmax_scale, cu_q, cu_k,
                                (char*)workspace, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_sparse_attn_fwd(const msa_shape* shape, const void* q, const void* k,
                               const void* v, const float* descale_qkv, float softmax_scale,
                               const int32_t* topk_idx, const int32_t* cu_q,
                               const int32_t* cu_k, msa_mode mode, void* workspace,
                               size_t ws_bytes, void* o, float* lse, hipStream_t stream) {
  msa_mode m;
  Geometry g;
  Layout L;
  msa_status st = prep(shape, mode, workspace, ws_bytes, &m, &g, &L);
  if (st != MSA_OK) return st;
  const msa_shape& s = *shape;
  if (!topk_idx || !cu_q || !cu_k) return MSA_ERR_NULL;
  if ((s.total_q > 0 && !q) || (s.total_k > 0 && (!k || !v))) return MSA_ERR_NULL;
  if (s.dtype == MSA_FP8_E4M3 && !descale_qkv) return MSA_ERR_NULL;
  hipError_t e;
  if (m == MSA_KV_OUTER) {
    e = launch_plan(s, g, L, topk_idx, cu_q, cu_k, (char*)workspace, stream);
    if (e == hipSuccess)
      e = launch_attn_kv(s, g, L, q, k, v, descale_qkv, softmax_scale, cu_q, cu_k,
                         (char*)workspace, stream);
  } else {
    if (g.splits == 1 && s.total_q > 0 && !o) return MSA_ERR_NULL;
    e = launch_attn_q(s, g, L, q, k, v, descale_qkv, softmax_scale, topk_idx, cu_q, cu_k,
                      (char*)workspace, o, lse, stream);
  }
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}

msa_status msa_combine(const msa_shape* shape, msa_mode mode, const void* workspace,
                       size_t ws_bytes, void* o, float* lse, hipStream_t stream) {
  msa_mode m;
  Geometry g;
  Layout L;
  msa_status st = prep(shape, mode, workspace, ws_bytes, &m, &g, &L);
  if (st != MSA_OK) return st;
  if (m == MSA_Q_OUTER && g.splits == 1) return MSA_OK;
  if (shape->total_q > 0 && !o) return MSA_ERR_NULL;
  hipError_t e = launch_combine(*shape, g, L, (const char*)workspace, o, lse, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}


msa_status msa_sparse_attn_fwd_noalloc(const msa_shape* shape, const void* q, const void* k,
                                       const void* v, const float* descale_qkv,
                                       float softmax_scale, const int32_t* topk_idx,
                                       const int32_t* cu_q, const int32_t* cu_k, msa_mode mode,
                                       void* o, float* lse, hipStream_t stream) {
  msa_status st = check_shape(shape);
  if (st != MSA_OK) return st;
  msa_mode m;
  st = check_mode(*shape, mode, &m);
  if (st != MSA_OK) return st;
  const size_t need = layout(*shape, m).total;
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) {
    g_last_error = "the shape needs " + std::to_string(need) + " bytes of scratch, more than the " +
                   std::to_string((size_t)MSA_NOALLOC_SCRATCH_BYTES) + " the library holds";
    return MSA_ERR_WORKSPACE;
  }
  if (shape->total_q > 0 && !o) return MSA_ERR_NULL;
  void* ws = scratch_ptr();
  if (!ws) return MSA_ERR_LAUNCH;
  // the same two calls as the workspace form, on the static scratch (nothing in it needs to
  // start at zero: the plan and the Q-outer kernels write every value the later kernels read)
  st = msa_sparse_attn_fwd(shape, q, k, v, descale_qkv, softmax_scale, topk_idx, cu_q, cu_k, m,
                           ws, MSA_NOALLOC_SCRATCH_BYTES, o, lse, stream);
  if (st != MSA_OK) return st;
  return msa_combine(shape, m, ws, MSA_NOALLOC_SCRATCH_BYTES, o, lse, stream);
}

msa_status msa_probe_read(const void* buf, size_t working_set_bytes, size_t total_bytes,
                          float* sink, hipStream_t stream) {
  if (!buf || !sink) return MSA_ERR_NULL;
  const size_t min_ws = (size_t)kProbeGrid * 4096;
  if (working_set_bytes < min_ws || working_set_bytes % 4096 != 0 || total_bytes < min_ws)
    return MSA_ERR_SHAPE;
  const hipError_t e = launch_probe_read(buf, working_set_bytes, total_bytes, sink, stream);
  if (e != hipSuccess) {
    fail_launch(e);
    return MSA_ERR_LAUNCH;
  }
  return MSA_OK;
}


}  // extern "C"
