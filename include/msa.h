/*
 * msa.h - C ABI of libmsa: MiniMax-style block-sparse GQA attention on AMD MI355X (gfx950).
 *
 * The operator ("Kernel optimization for MiniMax M3 on NVIDIA Blackwell", summary section)
 * cuts the KV sequence into 128-token blocks; an index branch scores the blocks for every
 * GQA group and keeps the top-K; a main branch computes exact attention over only the
 * selected blocks. This library runs the three steps as separate calls:
 *
 *   msa_index_topk       index branch: max-pooled proxy scores + top-K, local block forced
 *   msa_index_topk_fp8   the same on fp8 e4m3 proxies (8-bit MFMA scoring)
 *   msa_index_topk_mxfp4 the same on 4-bit MXFP4 proxies (scaled 4-bit MFMA scoring)
 *   msa_select_tiles     per-Q-tile lists from block representatives (R1 / R4 selectors)
 *   msa_sparse_attn_fwd  main branch: KV-outer partials (or Q-outer output) over the lists
 *   msa_combine          log-sum-exp merge of the per-slot partials into O and LSE
 *   msa_sparse_attn_bwd  main-branch backward: dQ, dK, dV over the selected blocks
 *   msa_proxy_attn_bwd   proxy backward: gradients of the proxies toward the main weights
 *   msa_train_bwd        both backward passes in one call
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers allocated and owned by the caller; the library never
 *    allocates, frees, synchronises, or copies device memory to the host. Work is enqueued on
 *    `stream` (NULL = the default stream) and the call returns without waiting.
 *  - Layouts are dense row-major. Q is [total_q, hq, d]; K and V are [total_k, hkv, d];
 *    q_idx is [total_q, hkv, dp]; k_idx is [total_k, hkv, dp]. Query head h belongs to KV
 *    group h / (hq / hkv), so the heads of one group are adjacent.
 *  - Variable-length batches: cu_q and cu_k are DEVICE int32 arrays of batch + 1
 *    non-decreasing offsets (cu[0] = 0, cu[batch] = total). Sequence s owns query rows
 *    [cu_q[s], cu_q[s+1]) and key rows [cu_k[s], cu_k[s+1]). Query i of a sequence with N
 *    queries and Nk keys sits at position pos = Nk - N + i (bottom-right alignment), and its
 *    local block is floor(pos / block). Each sequence must satisfy N <= max_q and
 *    Nk <= max_k; the library cannot check device-side values (no device-to-host copy).
 *  - Errors: argument checks run on the host before anything is enqueued; a non-OK status
 *    means nothing was launched. MSA_ERR_LAUNCH means a kernel launch failed (the HIP error
 *    text is in msa_last_error(), kept per thread).
 *  - Determinism: identical inputs give bitwise-identical outputs (no floating-point atomics;
 *    fixed reduction orders).
 */
#ifndef MSA_H
#define MSA_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,       /* a required pointer is NULL */
  MSA_ERR_SHAPE = 2,      /* sizes outside what this build supports, or inconsistent */
  MSA_ERR_DTYPE = 3,      /* unknown dtype */
  MSA_ERR_WORKSPACE = 4,  /* workspace pointer NULL or smaller than msa_workspace_size() */
  MSA_ERR_MODE = 5,       /* mode value unknown or not allowed for these shapes */
  MSA_ERR_LAUNCH = 6      /* a HIP kernel launch failed */
} msa_status;

typedef enum {
  MSA_BF16 = 0,       /* Q, K, V in bfloat16 */
  MSA_FP8_E4M3 = 1    /* Q, K, V in OCP fp8 e4m3fn with per-tensor fp32 descales */
} msa_dtype;

/* Schedule of the main branch ("Kernel optimization ...", section 1: the two structures).
 * KV_OUTER: each selected KV block is loaded once and every query that chose it is gathered
 * in; partial outputs are written and msa_combine merges them. Q_OUTER: each group of rows
 * that shares a list walks its blocks with an online softmax. AUTO picks by the nsb/N
 * bandwidth crossover (see msa_crossover). */
typedef enum { MSA_AUTO = 0, MSA_KV_OUTER = 1, MSA_Q_OUTER = 2 } msa_mode;

typedef struct {
  int32_t batch;    /* number of sequences, >= 1 */
  int32_t total_q;  /* rows of Q / q_idx: sum of per-sequence query counts, >= 0 */
  int32_t total_k;  /* rows of K / V / k_idx */
  int32_t max_q;    /* upper bound on any sequence's query count (sizes the schedule) */
  int32_t max_k;    /* upper bound on any sequence's key count */
  int32_t hq;       /* query heads */
  int32_t hkv;      /* KV heads (GQA groups); hq % hkv == 0, hq / hkv in {1, 2, 4, 8, 16} */
  int32_t d;        /* head dim: 128 */
  int32_t dp;       /* proxy (index) dim: 32 or 64; ignored when the index branch is unused */
  int32_t block;    /* KV block size: 128 */
  int32_t topk;     /* selected blocks per list: 1..16 */
  int32_t causal;   /* 1: key u visible to a query at position pos iff u <= pos */
  int32_t dtype;    /* msa_dtype of Q/K/V. Proxies are bf16 for msa_index_topk, e4m3fn
                       (with their own descales) for msa_index_topk_fp8 and MXFP4 (codes
                       and E8M0 group scales) for msa_index_topk_mxfp4 */
  int32_t list_q;   /* 1: per-query lists topk_idx [total_q, hkv, topk];
                       128: per-Q-tile lists [batch * ceil(max_q/128), hkv, topk], row
                       s * ceil(max_q/128) + t holds the list of queries [128t, 128t+128)
                       of sequence s ("Sparse Attention", Chapter 1, per-Q-tile selection) */
} msa_shape;

/* Layout of the workspace regions, for tests and tools. Offsets are in bytes from the start
 * of the workspace; a region of size 0 is unused. */
typedef struct {
  size_t counters;     /* int32[64]; [0] = number of (query-group, block) entries E */
  size_t masks;        /* uint64 bitmaps, bucket-major. Bucket (s, g, r, b) covers the
                          queries [64 W r, 64 W (r + 1)) of sequence s for group g and block b
                          (W = words_per_bucket); its word w has bit i set when query
                          64 (W r + w) + i listed block b */
  size_t offsets;      /* int32 exclusive scan of the bitmap popcounts, n_words + 1 values */
  size_t scan_sums;    /* int32 scratch of the scan */
  size_t entry_q;      /* int32 [E]: query row of entry e; entries are sorted by
                          (sequence, group, query range r, block, query) */
  size_t entry_bucket; /* int32 [E]: bucket ((s * hkv + g) * n_ranges + r) * nb_max + b */
  size_t cmap;         /* int32 [total_q, hkv, slots]: partial index of each slot, -1 = none */
  size_t part_lse;     /* float [E, hq/hkv]: log-sum-exp of each partial */
  size_t part_l;       /* float [E, hq/hkv]: sum of each partial's softmax weights (as rounded
                          for the PV product), each taken relative to the partial's maximum and
                          divided by a positive factor that part_o carries too (bf16: 1; fp8:
                          the V descale, part_o holding the output against the raw e4m3 values
                          of V); 1 where the partial output is already normalised */
  size_t part_o;       /* bf16, E * hq/hkv rows of d: partial output before normalisation,
                          i.e. the partial's attention output times part_l ("Kernel
                          optimization ...", section 2: unnormalised accumulators, normalised
                          in the combine). Row p = e * (hq/hkv) + head is stored in groups of 8
                          rows: dims 8c .. 8c+7 of row p at byte ((p / 8) * 16 + c) * 128 +
                          (p % 8) * 16, so that dims 8c .. 8c+7 of 8 consecutive rows fill one
                          128-byte line (the rows are padded to a multiple of 8) */
  size_t v_wide;       /* KV-outer: bf16 V^T of every (kv head, key block), the PV operand
                          of the attention kernels (e4m3 V widened exactly): block b of
                          sequence s and kv head h is the 128 x 128 array
                          [h][cu_k[s] / 128 + s + b][d][key], keys past the sequence's end
                          zero; hkv * (ceil(total_k / 128) + batch) blocks. Written by
                          msa_sparse_attn_fwd before its attention kernel (size 0 for
                          Q-outer) */
  size_t total;        /* bytes needed */
  int32_t slots;       /* slots per (query, group) in cmap */
  int32_t n_words;     /* bitmap words (0 for Q-outer) */
  int32_t w_max;       /* bitmap words per (sequence, group, block): ceil(max_q / 64) */
  int32_t nb_max;      /* blocks per sequence bound */
  int32_t words_per_bucket; /* bitmap words per bucket */
  int32_t n_ranges;    /* query ranges per sequence */
} msa_workspace_layout;

/* ---- host-only queries (no GPU needed) ---------------------------------------------- */

/* Bytes of workspace msa_sparse_attn_fwd and msa_combine need for `shape` under `mode`.
 * KV-outer holds the inverted index (bitmaps, scan, entry list, combine map) and E bf16
 * partials of (hq/hkv) x d plus fp32 LSEs and weight sums, E <= total_q * hkv * topk; with
 * fp8 Q/K/V also a bf16 copy of V (total_k * hkv * d * 2 bytes). Errors: NULL, SHAPE, DTYPE,
 * MODE. */
msa_status msa_workspace_size(const msa_shape* shape, msa_mode mode, size_t* bytes);

/* Region offsets of that workspace (same errors). */
msa_status msa_workspace_layout_of(const msa_shape* shape, msa_mode mode,
                                   msa_workspace_layout* out);

/* Bytes of workspace msa_index_topk needs: non-zero only for short-query calls (max_q <= 16),
 * where the key range of every query is scored in chunks by separate workgroups and the
 * chunks' partial top-K lists (8 bytes per entry, 16 entries per chunk) are merged. */
msa_status msa_index_workspace_size(const msa_shape* shape, size_t* bytes);

/* The schedule msa_sparse_attn_fwd runs for `mode` (AUTO resolved). Per-Q-tile lists always
 * run Q-outer; otherwise AUTO runs KV-outer iff nsb_max / total_q < msa_crossover(), where
 * nsb_max = min(batch * hkv * ceil(max_k/block), total_q * hkv * topk) bounds the distinct
 * selected blocks from the shape alone. */
msa_status msa_resolve_mode(const msa_shape* shape, msa_mode mode, msa_mode* chosen);

/* Bandwidth-roofline crossover X ("Kernel optimization ...", section 1 and appendix):
 * KV-outer is the faster schedule when nsb / N < X. KV-outer moves each selected block once
 * plus, per query, Q, its partials (written and read back) and O through HBM; Q-outer
 * re-reads every list's blocks through the cache at bw_cache. With e = bytes per Q/K/V
 * element, partials bf16 and LSE fp32, per query token:
 *   kv_per_n = hq*d*e + hq*topk*(2*2*d + 2*4) + hq*d*2 ;  q_per_n = hkv*topk*2*block*d*e + hq*d*(e+2)
 *   X = (q_per_n * bw_hbm / bw_cache - kv_per_n) / (2*block*d*e).
 * bw_* in any common unit; bw_cache = 0 selects the MI355X default ratio 2.32, measured (the
 * ratio at which this model reproduces the crossover of the two schedules timed over block
 * reuse on MI355X; its last-level cache alone reads 1.32x the HBM rate). AUTO uses it. */
msa_status msa_crossover(const msa_shape* shape, double bw_hbm, double bw_cache, double* x);

const char* msa_status_string(msa_status st);
const char* msa_last_error(void);

/* ---- device calls ----------------------------------------------------------------------- */

/* Index branch ("Flash-MSA: accelerating million-token training", proxy forward; "Kernel
 * optimization ...", summary). For every query row i and group g: for each visible block j
 * other than the local block c, s_j = max over keys u of block j (u < Nk; u <= pos if causal)
 * of the fp32 dot product q_idx[i,g,:] . k_idx[u,g,:]; s_c = +inf. topk_idx[i,g,:] receives
 * the first min(topk, #visible) blocks by (s descending, block index ascending) - the local
 * block in slot 0 - and -1 in unused slots. topk_score (nullable) receives the matching
 * scores (+inf for the local block, -inf for unused slots).
 * In: q_idx, k_idx bf16 (layouts above), cu_q, cu_k. Out: topk_idx [total_q, hkv, topk]
 * int32, topk_score [total_q, hkv, topk] fp32. workspace: msa_index_workspace_size() bytes
 * (may be NULL when that size is 0), else MSA_ERR_WORKSPACE. Requires list_q == 1,
 * dp in {32, 64}; short-query calls (max_q <= 16) take max_k <= 2^21 keys. */
msa_status msa_index_topk(const msa_shape* shape, const void* q_idx, const void* k_idx,
                          const int32_t* cu_q, const int32_t* cu_k, int32_t* topk_idx,
                          float* topk_score, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Low-precision index scoring ("Sparse Attention", Chapter 4: a scorer that compares
 * quantised index vectors, token by token, and keeps each block's largest score; the pages
 * use 4-bit inputs, as msa_index_topk_mxfp4 does; this call takes OCP fp8 e4m3fn). The same
 * selection, arguments, workspace and errors as msa_index_topk, except:
 *  - q_idx and k_idx hold e4m3fn codes; descale_idx is a DEVICE float[2] with their positive
 *    per-tensor descales (proxy value = code * descale), NULL: MSA_ERR_NULL.
 *  - Each proxy dot product is the exact products of the codes summed in fp32 (an 8-bit MFMA
 *    per 32 x 32 score tile for prefill); block scores, and topk_score, are max(q.k) times
 *    descale_idx[0] * descale_idx[1]. */
msa_status msa_index_topk_fp8(const msa_shape* shape, const void* q_idx, const void* k_idx,
                              const float* descale_idx, const int32_t* cu_q, const int32_t* cu_k,
                              int32_t* topk_idx, float* topk_score, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/* 4-bit index scoring ("Sparse Attention", Chapter 4: the FP4 scorer, 4-bit index vectors
 * with scales prepared before the call; one score per (query, key), the block keeps its
 * largest). The format is OCP MXFP4, the 4-bit form gfx950's scaled MFMA takes. The same
 * selection, arguments, workspace and errors as msa_index_topk, except:
 *  - q_idx [total_q, hkv, dp / 2] and k_idx [total_k, hkv, dp / 2] bytes hold E2M1 codes,
 *    element 2i of a row in the low nibble of byte i;
 *  - q_scale [total_q, hkv, dp / 32] and k_scale [total_k, hkv, dp / 32] (DEVICE uint8) hold
 *    the E8M0 scale of elements 32b .. 32b + 31 of each row (value 2^(code - 127); code 255,
 *    NaN in the format, is not checked and gives undefined scores); NULL with a non-empty
 *    side: MSA_ERR_NULL.
 *  - A proxy element is its code's value times its group's scale. Per group the products are
 *    exact and summed exactly; only the sum over the dp / 32 groups rounds (fp32), so scores
 *    are exact whenever the exact value is an fp32 number. Block scores, and topk_score, are
 *    max(q.k), unscaled. */
msa_status msa_index_topk_mxfp4(const msa_shape* shape, const void* q_idx,
                                const uint8_t* q_scale, const void* k_idx,
                                const uint8_t* k_scale, const int32_t* cu_q, const int32_t* cu_k,
                                int32_t* topk_idx, float* topk_score, void* workspace,
                                size_t ws_bytes, hipStream_t stream);

/* Per-Q-tile block selectors R1 and R4 ("Sparse Attention", Chapter 4: one or four
 * representatives). Every 128-query tile of a sequence and every 128-key block is summarised,
 * per head, by the mean of its token vectors (reps = 1) or by the means of its four
 * consecutive 32-token groups (reps = 4); a ragged tile or block averages the tokens it has
 * and an empty group takes part in no comparison. A block's score for a (tile, group) is the
 * largest dot product between a query representative of any query head of the group and a
 * key representative of the block (the raw values: no softmax scale). With causal = 1 a block
 * is visible to a tile when its first key is not after the tile's last query position
 * (bottom-right aligned); no block is forced. Writes the per-tile lists the per-Q-tile
 * attention reads: lists [batch * ceil(max_q / 128), hkv, topk] int32, row
 * s * ceil(max_q / 128) + t, the blocks by score descending then block ascending, -1 where
 * fewer blocks are visible (and for rows past a sequence's tiles); scores (nullable) the same
 * shape, fp32, -inf at -1 slots. Requires list_q == 128 and bf16 Q and K
 * (MSA_ERR_DTYPE otherwise); q [total_q, hq, d], k [total_k, hkv, d]; reps in {1, 4}.
 * workspace: msa_select_workspace_size() bytes (fp32 representatives and block scores). */
msa_status msa_select_workspace_size(const msa_shape* shape, int reps, size_t* bytes);
msa_status msa_select_tiles(const msa_shape* shape, int reps, const void* q, const void* k,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t* lists,
                            float* scores, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/* Main branch ("Kernel optimization ...", summary and section 2; "Sparse Attention",
 * Chapters 1 and 5). Every query head attends, with its own softmax, to the union of the
 * keys of its group's selected blocks (key u of block b is u = block*b + offset, u < Nk, and
 * u <= pos if causal); scores are softmax_scale * q.k (times descale_q * descale_k for fp8),
 * values are scaled by descale_v. Lists: topk_idx as described for list_q; entries outside
 * [0, ceil(Nk/block)), repeated entries, and (causal) blocks wholly after the query are
 * ignored.
 * KV_OUTER: builds the block -> query inverted index in the workspace and a transposed bf16
 * copy of V (v_wide, the PV operand layout), then one kernel loads each selected block once
 * and writes, for every (query-group, block) entry, contiguously
 * in entry order: the UNNORMALISED partial output (bf16, part_o: the block's attention output
 * times its weight sum), the weight sum (fp32, part_l) and the partial's LSE (fp32,
 * part_lse); see msa_workspace_layout. msa_combine, which must follow on the same stream,
 * divides by part_l and merges by LSE. `o` and `lse` are not touched.
 * Q_OUTER: writes O (same dtype as the result of msa_combine: bf16 [total_q, hq, d]) and LSE
 * (fp32 [total_q, hq]) directly, or - when the schedule splits long lists - partials that
 * msa_combine merges. Calling msa_combine after Q_OUTER is always valid.
 * descale_qkv: DEVICE float[3] (dq, dk, dv) for fp8; NULL for bf16. The workspace must hold
 * msa_workspace_size(shape, mode) bytes and stay untouched until msa_combine has run. */
msa_status msa_sparse_attn_fwd(const msa_shape* shape, const void* q, const void* k,
                               const void* v, const float* descale_qkv, float softmax_scale,
                               const int32_t* topk_idx, const int32_t* cu_q,
                               const int32_t* cu_k, msa_mode mode, void* workspace,
                               size_t ws_bytes, void* o, float* lse, hipStream_t stream);

/* KV-outer halves of msa_sparse_attn_fwd, for timing the inverted-index build and the
 * attention kernels separately (msa_attn_main: the transposed V copy, then the attention
 * kernel). msa_plan(...) followed by msa_attn_main(...) with the same arguments is exactly
 * msa_sparse_attn_fwd(..., MSA_KV_OUTER, ...). */
msa_status msa_plan(const msa_shape* shape, const int32_t* topk_idx, const int32_t* cu_q,
                    const int32_t* cu_k, void* workspace, size_t ws_bytes, hipStream_t stream);
msa_status msa_attn_main(const msa_shape* shape, const void* q, const void* k, const void* v,
                         const float* descale_qkv, float softmax_scale, const int32_t* cu_q,
                         const int32_t* cu_k, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/* Combine ("Sparse Attention", Chapter 5, partial outputs and combine; "Kernel optimization
 * ...", section 2: the combine kernel gathers through the index map). For every query row and
 * head: LSE = log sum_slot exp(lse_slot) over the valid slots (max-shifted), O = sum_slot
 * exp(lse_slot - LSE) * O_slot; with no valid slot, O = 0 and LSE = -inf. Reads the
 * workspace written by msa_sparse_attn_fwd with the same shape and mode. Out: o bf16
 * [total_q, hq, d], lse fp32 [total_q, hq] (lse may be NULL). A no-op when the Q-outer
 * schedule already wrote O. */
msa_status msa_combine(const msa_shape* shape, msa_mode mode, const void* workspace,
                       size_t ws_bytes, void* o, float* lse, hipStream_t stream);

/* Read-bandwidth probe for the schedule choice ("Kernel optimization ...", section 1 and
 * appendix: the KV-outer / Q-outer crossover scales with the measured ratio of cache to HBM
 * bandwidth). Reads total_bytes of the device buffer `buf` by sweeping its first
 * working_set_bytes over and over, each sweep one coalesced pass of 1024 workgroups of 4 KiB
 * each, and writes 1024 * 256 floats (checksums) to the device buffer `sink`. A working set
 * larger than the last-level cache (256 MB on MI355X) streams from HBM, one within it from the
 * cache. Time it with events on `stream`. Requires working_set_bytes >= 4 MiB and a multiple of
 * 4096, total_bytes >= 4 MiB (read in whole passes of 4 MiB); SHAPE otherwise, NULL for a
 * missing buffer. */
msa_status msa_probe_read(const void* buf, size_t working_set_bytes, size_t total_bytes,
                          float* sink, hipStream_t stream);

/* Allocation-free form of the main branch, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Runs msa_sparse_attn_fwd followed by msa_combine with the same arguments, its workspace
 * being a scratch array the library holds on each device (MSA_NOALLOC_SCRATCH_BYTES bytes per
 * device, kept until the process ends), so `o` and `lse` (nullable) receive the final O and LSE
 * whichever schedule `mode` resolves to. Calls no allocating routine. Errors: those of the two
 * calls, and MSA_ERR_WORKSPACE (with the byte counts in msa_last_error) when
 * msa_workspace_size(shape, mode) exceeds MSA_NOALLOC_SCRATCH_BYTES (a tiny prefill of 2048
 * queries with 16 heads and topK 4 needs about 36 MB; 64 decode requests well under 8 MB).
 * Every call on one device shares that device's scratch: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be serialised by the caller. */
#define MSA_NOALLOC_SCRATCH_BYTES (64u << 20)
msa_status msa_sparse_attn_fwd_noalloc(const msa_shape* shape, const void* q, const void* k,
                                       const void* v, const float* descale_qkv,
                                       float softmax_scale, const int32_t* topk_idx,
                                       const int32_t* cu_q, const int32_t* cu_k, msa_mode mode,
                                       void* o, float* lse, hipStream_t stream);

/* Main-branch backward ("Flash-MSA: accelerating million-token training": the selected block
 * ids and the main branch's LSE are kept for the backward; the gradients are those of the
 * exact attention over each query's union of selected keys, as in msa_sparse_attn_fwd; the
 * lists themselves are not differentiated). With P = exp(softmax_scale q.k - LSE) over the
 * visible keys and D = sum_d dO O per (query, head):
 *   dV_u = sum P dO,  dS = P (dO.v_u - D),  dQ = softmax_scale sum_u dS k_u,
 *   dK_u = softmax_scale sum dS q  (sums over the query heads of u's group that see u).
 * bf16 only (DTYPE otherwise). In: q, o, dout bf16 [total_q, hq, d]; k, v bf16
 * [total_k, hkv, d]; lse fp32 [total_q, hq] as written by msa_combine (natural log); lists,
 * cu_q, cu_k as for msa_sparse_attn_fwd. Out (fp32, written, not accumulated): dq
 * [total_q, hq, d]; dk, dv [total_k, hkv, d]. Every row of dq is written (zero for rows with
 * no visible key or in no sequence); dk and dv rows of keys in a sequence are written (zero
 * for keys no query sees), other rows are not touched. Deterministic: no atomics. Workspace:
 * msa_bwd_workspace_size bytes (the KV-outer plan plus bf16 dQ partials of every
 * (query-group, block) entry: E x hq/hkv x d x 2 bytes). */
msa_status msa_bwd_workspace_size(const msa_shape* shape, size_t* bytes);
msa_status msa_sparse_attn_bwd(const msa_shape* shape, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dout,
                               float softmax_scale, const int32_t* topk_idx,
                               const int32_t* cu_q, const int32_t* cu_k, void* workspace,
                               size_t ws_bytes, float* dq, float* dk, float* dv,
                               hipStream_t stream);

/* Proxy (index-branch) backward ("Flash-MSA: accelerating million-token training": the proxy
 * gradients need the proxy and the main attention probabilities together, and the proxy LSE
 * is recomputed over the sparse keys in the backward; the objective itself is not printed on
 * the pages, and this library takes the following one). Per query row and KV group, over the
 * same selected keys as msa_sparse_attn_fwd: T = the main weights exp(softmax_scale q.k - LSE)
 * averaged over the group's heads (held fixed), Pp = softmax(proxy_scale q_idx.k_idx), and the
 * gradients of sum KL(T || Pp): dz = proxy_scale (Pp - T), dq_idx = sum_u dz k_idx_u,
 * dk_idx_u = sum dz q_idx. bf16 only, dp in {32, 64}. In: q bf16 [total_q, hq, d], k bf16
 * [total_k, hkv, d], q_idx / k_idx bf16 proxies, lse fp32 [total_q, hq] (the forward's); lists
 * as for msa_sparse_attn_fwd. Out (fp32, written): dq_idx [total_q, hkv, dp] (every row),
 * dk_idx [total_k, hkv, dp] (rows of keys in a sequence); lse_proxy fp32 [total_q, hkv] when
 * not NULL (natural log, -inf for a row with no visible key). Deterministic. Workspace:
 * msa_proxy_bwd_workspace_size bytes. */
msa_status msa_proxy_bwd_workspace_size(const msa_shape* shape, size_t* bytes);
msa_status msa_proxy_attn_bwd(const msa_shape* shape, const void* q, const void* k,
                              const void* q_idx, const void* k_idx, const float* lse,
                              float softmax_scale, float proxy_scale, const int32_t* topk_idx,
                              const int32_t* cu_q, const int32_t* cu_k, void* workspace,
                              size_t ws_bytes, float* dq_idx, float* dk_idx, float* lse_proxy,
                              hipStream_t stream);

/* The whole backward of a training step in one call ("Flash-MSA ...": main and proxy
 * gradients): msa_sparse_attn_bwd then msa_proxy_attn_bwd on the same arguments, enqueued on
 * `stream` one after the other and sharing one workspace of msa_train_bwd_workspace_size
 * bytes (the larger of the two). Same inputs, outputs, errors and conventions as those two
 * calls, and bitwise the same results. */
msa_status msa_train_bwd_workspace_size(const msa_shape* shape, size_t* bytes);
msa_status msa_train_bwd(const msa_shape* shape, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dout, float softmax_scale,
                         const void* q_idx, const void* k_idx, float proxy_scale,
                         const int32_t* topk_idx, const int32_t* cu_q, const int32_t* cu_k,
                         void* workspace, size_t ws_bytes, float* dq, float* dk, float* dv,
                         float* dq_idx, float* dk_idx, float* lse_proxy, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
