"""Plain fp64 CPU oracle of MiniMax-style block-sparse GQA attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path and imports
nothing from it; it is slow on purpose and written to be checked against the pages by eye.

What it computes (the plain definition the fast path must reach, up to rounding order):

* Index branch ("Flash-MSA: accelerating million-token training", the paragraphs on the
  proxy forward; "Kernel optimization for MiniMax M3 on NVIDIA Blackwell", summary section):
  per (query, KV group) a proxy score for every visible 128-token KV block, the maximum of
  the proxy dot products q_idx . k_idx over the block's keys (max-pooling, causal within the
  chunk), the query's own local block forced to +inf, then the top-K blocks.
* Main branch ("Kernel optimization ...", summary; "Sparse Attention", Chapter 1): exact
  softmax attention of every query head over the union of the keys of its group's selected
  blocks; unselected keys get zero weight; each head has its own softmax ("Sparse
  Attention", Chapter 2, GQA section).
* Partials and combine ("Sparse Attention", Chapter 5, partial outputs and combine): the
  same attention restricted to one selected block gives a partial output and its
  log-sum-exp; merging the partials with weights exp(lse_slot - LSE) gives the full result.

Readings adopted where the pages are silent (each one is listed in the design notes):
positions are bottom-right aligned (pos = Nk - N + i); a query's local block is
pos // block; the forced local block takes one of the K slots; ties between equal proxy
scores go to the lower block index; a query with fewer than K visible blocks gets the
rest of its slots padded with -1; slots are ordered local first, then by score
descending, then block index ascending; repeated or out-of-range blocks in a given list
count once or not at all (the union of valid blocks); a query with no visible key gets
O = 0 and LSE = -inf; LSE is the natural-log log-sum-exp of the scaled scores.

Parity status: every function here is pinned by the CPU tests (dense and local-only
special cases against torch's scaled_dot_product_attention, brute-force exact selection on
small-integer proxies, the streaming insertion sort of the proxy page, invariants, the
combine identity, and the worked list example of "Sparse Attention", Chapter 2).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf
POS_INF = np.inf


# --------------------------------------------------------------------------- positions

def query_positions(n_q: int, n_k: int) -> np.ndarray:
    """Bottom-right aligned positions pos(i) = Nk - N + i (prefill N = Nk gives pos = i;
    decode N = 1 gives pos = Nk - 1)."""
    return n_k - n_q + np.arange(n_q, dtype=np.int64)


def n_blocks(n_k: int, block: int) -> int:
    return -(-n_k // block)


# --------------------------------------------------------------------------- index branch

def proxy_block_scores(q_idx: np.ndarray, k_idx: np.ndarray, block: int, causal: bool,
                       rows: np.ndarray | None = None, n_q_chunk: int = 512) -> np.ndarray:
    """Max-pooled proxy block scores of one sequence.

    q_idx [N, Hkv, dp], k_idx [Nk, Hkv, dp] (fp64); ``rows`` picks query rows (default all).
    Returns s [n, Hkv, nb] fp64 with s_j = max over keys u of block j (u < Nk, and
    u <= pos(i) if causal) of q_idx[i, g] . k_idx[u, g]; -inf where block j has no visible
    key; +inf at the local block c = pos(i) // block when it exists (the proxy page forces
    the local score to infinity).
    """
    n_q, hkv, _ = q_idx.shape
    n_k = k_idx.shape[0]
    nb = n_blocks(n_k, block)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = query_positions(n_q, n_k)[rows]
    n = rows.size
    out = np.full((n, hkv, nb), NEG_INF)
    key_pos = np.arange(nb * block, dtype=np.int64)
    for g in range(hkv):
        kg = k_idx[:, g, :]
        for i0 in range(0, n, n_q_chunk):
            i1 = min(n, i0 + n_q_chunk)
            dots = np.full((i1 - i0, nb * block), NEG_INF)
            dots[:, :n_k] = q_idx[rows[i0:i1], g, :] @ kg.T
            if causal:
                dots[key_pos[None, :] > pos[i0:i1, None]] = NEG_INF
            out[i0:i1, g, :] = dots.reshape(i1 - i0, nb, block).max(axis=2)
    local = pos // block
    has_local = (local >= 0) & (local < nb)
    r = np.nonzero(has_local)[0]
    out[r, :, local[r]] = POS_INF
    return out


def select_topk(scores: np.ndarray, topk: int) -> np.ndarray:
    """Top-K block ids per (query, group) from max-pooled scores [N, Hkv, nb].

    Blocks are ranked by (score descending, block index ascending); -inf (invisible) blocks
    are never selected; unused slots hold -1. The forced local block (+inf) lands in slot 0.
    """
    n_q, hkv, nb = scores.shape
    out = np.full((n_q, hkv, topk), -1, dtype=np.int32)
    if nb == 0:
        return out
    # a stable sort on the negated score keeps lower block indices first among equal scores
    order = np.argsort(-scores, axis=2, kind="stable")
    take = min(topk, nb)
    sel = order[:, :, :take]
    val = np.take_along_axis(scores, sel, axis=2)
    out[:, :, :take] = np.where(val > NEG_INF, sel, -1).astype(np.int32)
    return out


def index_topk(q_idx: np.ndarray, k_idx: np.ndarray, block: int, topk: int,
               causal: bool, rows: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Index branch of one sequence: (topk_idx [n, Hkv, K] int32, scores [n, Hkv, nb])."""
    s = proxy_block_scores(q_idx, k_idx, block, causal, rows=rows)
    return select_topk(s, topk), s


# --------------------------------------------------------------------------- main branch

def _key_set(blocks: np.ndarray, n_k: int, block: int, pos: int, causal: bool) -> np.ndarray:
    """Sorted key positions of the union of the valid selected blocks of one query."""
    nb = n_blocks(n_k, block)
    uniq = np.unique(blocks[(blocks >= 0) & (blocks < nb)])
    if uniq.size == 0:
        return np.zeros(0, dtype=np.int64)
    keys = (uniq[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    keys = keys[keys < n_k]
    if causal:
        keys = keys[keys <= pos]
    return keys


def attend(qh: np.ndarray, kk: np.ndarray, vv: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of rows qh [R, D] over keys kk [S, D], values vv [S, D].
    Returns (O [R, D], LSE [R]); with S = 0, O = 0 and LSE = -inf."""
    r, d = qh.shape
    if kk.shape[0] == 0:
        return np.zeros((r, vv.shape[1] if vv.ndim == 2 else d)), np.full(r, NEG_INF)
    x = scale * (qh @ kk.T)
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vv) / l
    return o, (m + np.log(l))[:, 0]


def lists_for_queries(lists: np.ndarray, n_q: int, list_q: int) -> np.ndarray:
    """Expand per-tile lists [ceil(N/list_q), Hkv, K] to per-query [N, Hkv, K]."""
    return lists[np.arange(n_q) // list_q]


def sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
                     scale: float, block: int, causal: bool,
                     rows: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Main branch of one sequence.

    q [N, Hq, D], k/v [Nk, Hkv, D], sel [N, Hkv, K] per-query block ids (fp64 inputs).
    Returns O [n, Hq, D], LSE [n, Hq] for the query rows ``rows`` (default: all)."""
    n_q, hq, _ = q.shape
    n_k, hkv, dv = v.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, hq, dv))
    lse = np.full((rows.size, hq), NEG_INF)
    for ri, i in enumerate(rows):
        for g in range(hkv):
            keys = _key_set(sel[i, g], n_k, block, int(pos[i]), causal)
            heads = slice(g * grp, (g + 1) * grp)
            o[ri, heads], lse[ri, heads] = attend(q[i, heads], k[keys, g], v[keys, g], scale)
    return o, lse


def partial_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
                      scale: float, block: int, causal: bool,
                      rows: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Per-slot partials of one sequence: attention restricted to the single block in each
    slot. Returns O_slot [n, Hq, K, D] (normalised) and lse_slot [n, Hq, K]. A slot whose
    block is -1, out of range, already listed in an earlier slot, or has no visible key is
    empty: O_slot = 0, lse_slot = -inf."""
    n_q, hq, _ = q.shape
    n_k, hkv, dv = v.shape
    kk = sel.shape[2]
    grp = hq // hkv
    nb = n_blocks(n_k, block)
    pos = query_positions(n_q, n_k)
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, hq, kk, dv))
    lse = np.full((rows.size, hq, kk), NEG_INF)
    for ri, i in enumerate(rows):
        for g in range(hkv):
            heads = slice(g * grp, (g + 1) * grp)
            seen = set()
            for slot in range(kk):
                b = int(sel[i, g, slot])
                if b < 0 or b >= nb or b in seen:
                    continue
                seen.add(b)
                keys = _key_set(np.array([b]), n_k, block, int(pos[i]), causal)
                o[ri, heads, slot], lse[ri, heads, slot] = attend(q[i, heads], k[keys, g],
                                                                  v[keys, g], scale)
    return o, lse


def combine(o_slot: np.ndarray, lse_slot: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Merge partials by log-sum-exp: LSE = log sum_slot exp(lse_slot) (max-shifted),
    O = sum_slot exp(lse_slot - LSE) O_slot. Slots with lse = -inf carry no weight; if every
    slot is empty, O = 0 and LSE = -inf. o_slot [..., K, D], lse_slot [..., K]."""
    m = lse_slot.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_slot - m_safe)                    # exp(-inf) = 0 for empty slots
    tot = w.sum(axis=-1, keepdims=True)
    lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, tot)))
    wn = np.where(empty, 0.0, w / np.where(empty, 1.0, tot))
    o = np.einsum("...k,...kd->...d", wn, o_slot)
    return o, lse[..., 0]
