"""Plain fp64 CPU oracle of the proxy (index-branch) backward of block-sparse GQA attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path.

"Flash-MSA: accelerating million-token training": the proxy gradients need both the proxy
and the main attention probabilities (a combined pass), the proxy log-sum-exp is recomputed
over the sparse (selected) keys in the backward, and the block ids are cached from the proxy
forward. The pages do not print the proxy objective; the reading taken here: per query row i
and KV group g, over the same key set S(i, g) the main branch attends to,

    T_iu   = (1/G) sum_(h in g) P_main[i, h, u]         (main weights, averaged over heads;
                                                          held fixed: no gradient to Q, K)
    z_iu   = q_idx_i . k_idx_u,  Pp_iu = exp(tau_p z_iu - LSEp_i),  LSEp_i = log sum_u e^(tau_p z)
    loss   = sum_(i, g) KL(T_i || Pp_i) = sum T log(T / Pp)
    dz_iu  = tau_p (Pp_iu - T_iu)
    dq_idx_i = sum_u dz_iu k_idx_u,   dk_idx_u = sum_i dz_iu q_idx_i.

Parity unpinned against the pages: they fix neither this objective nor any gradient value.
The pins (autograd of the same objective written densely, finite differences, the case
where the two distributions are equal) tie this code to the objective above, which is a
reading, not the pages' statement.
"""
from __future__ import annotations

import numpy as np

from oracle.msa_ref import _key_set, attend, query_positions


def proxy_backward(q: np.ndarray, k: np.ndarray, q_idx: np.ndarray, k_idx: np.ndarray,
                   sel: np.ndarray, scale: float, proxy_scale: float, block: int, causal: bool
                   ) -> tuple[np.ndarray, np.ndarray, float, np.ndarray]:
    """One sequence: q [N, Hq, D], k [Nk, Hkv, D], q_idx [N, Hkv, dp], k_idx [Nk, Hkv, dp],
    sel [N, Hkv, K]. Returns (dq_idx [N, Hkv, dp], dk_idx [Nk, Hkv, dp], loss, LSEp [N, Hkv]).
    A (query, group) with no visible key contributes nothing (LSEp = -inf)."""
    n_q, hq, _ = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    dqi = np.zeros_like(q_idx)
    dki = np.zeros_like(k_idx)
    lsep = np.full((n_q, hkv), -np.inf)
    loss = 0.0
    for i in range(n_q):
        for g in range(hkv):
            keys = _key_set(sel[i, g], n_k, block, int(pos[i]), causal)
            if keys.size == 0:
                continue
            heads = slice(g * grp, (g + 1) * grp)
            kk = k[keys, g]
            _, li = attend(q[i, heads], kk, kk, scale)                  # main LSE per head
            t = np.mean(np.exp(scale * (q[i, heads] @ kk.T) - li[:, None]), axis=0)
            z = proxy_scale * (k_idx[keys, g] @ q_idx[i, g])
            m = np.max(z)
            lp = m + np.log(np.sum(np.exp(z - m)))
            pp = np.exp(z - lp)
            lsep[i, g] = lp
            pos_t = t > 0
            loss += float(np.sum(t[pos_t] * (np.log(t[pos_t]) - np.log(pp[pos_t]))))
            dz = proxy_scale * (pp - t)
            dqi[i, g] = dz @ k_idx[keys, g]
            np.add.at(dki[:, g], keys, np.outer(dz, q_idx[i, g]))
    return dqi, dki, loss, lsep


def run_case(case, lists: np.ndarray, proxy_scale: float):
    """The proxy backward of a whole seeded case on per-query ``lists`` [Tq, Hkv, K].
    Returns (dq_idx [Tq, Hkv, dp], dk_idx [Tk, Hkv, dp], loss, LSEp [Tq, Hkv])."""
    from synth.msa_inputs import widen
    cfg = case.cfg
    dsq, dsk, _ = case.descale
    q, k = widen(case.q, dsq), widen(case.k, dsk)
    dqi_s, dki_s = case.idx_descale
    qi, ki = widen(case.q_idx, dqi_s), widen(case.k_idx, dki_s)
    dq = np.zeros_like(qi)
    dk = np.zeros_like(ki)
    lsep = np.full((case.total_q, cfg.hkv), -np.inf)
    loss = 0.0
    for s in range(len(case.cu_q) - 1):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        k0, k1 = int(case.cu_k[s]), int(case.cu_k[s + 1])
        if q1 == q0:
            continue
        a, b, l, lp = proxy_backward(q[q0:q1], k[k0:k1], qi[q0:q1], ki[k0:k1], lists[q0:q1],
                                     case.softmax_scale, proxy_scale, cfg.block, cfg.causal)
        dq[q0:q1], dk[k0:k1], lsep[q0:q1] = a, b, lp
        loss += l
    return dq, dk, loss, lsep


def _row_terms(q, k, q_idx, k_idx, keys, i, g, grp, scale, proxy_scale):
    """One (query, group): (dz over its key set, proxy LSE), as in proxy_backward."""
    heads = slice(g * grp, (g + 1) * grp)
    kk = k[keys, g]
    _, li = attend(q[i, heads], kk, kk, scale)
    t = np.mean(np.exp(scale * (q[i, heads] @ kk.T) - li[:, None]), axis=0)
    z = proxy_scale * (k_idx[keys, g] @ q_idx[i, g])
    m = np.max(z)
    lp = m + np.log(np.sum(np.exp(z - m)))
    return proxy_scale * (np.exp(z - lp) - t), lp


def proxy_rows_gradient(q, k, q_idx, k_idx, sel_rows, rows, scale, proxy_scale, block, causal):
    """dq_idx and the proxy LSE of the given query ``rows`` of one sequence only (a row's
    terms depend on its own list alone); sel_rows [R, Hkv, K]. The same formulas as
    proxy_backward. Returns (dq_idx [R, Hkv, dp], LSEp [R, Hkv])."""
    n_q, hq, _ = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    dqi = np.zeros((rows.size, hkv, q_idx.shape[2]))
    lsep = np.full((rows.size, hkv), -np.inf)
    for r, i in enumerate(rows):
        for g in range(hkv):
            keys = _key_set(sel_rows[r, g], n_k, block, int(pos[i]), causal)
            if keys.size == 0:
                continue
            dz, lsep[r, g] = _row_terms(q, k, q_idx, k_idx, keys, i, g, grp, scale, proxy_scale)
            dqi[r, g] = dz @ k_idx[keys, g]
    return dqi, lsep


def proxy_key_block_gradient(q, k, q_idx, k_idx, sel, g, b, scale, proxy_scale, block, causal):
    """dk_idx of the keys of block ``b`` of group ``g`` only: the sum over the queries whose
    list for g holds b of dz_iu q_idx_i, each query's dz over its own whole key set.
    Returns [n_b, dp] for the keys block*b .. min(block*(b+1), Nk) - 1."""
    n_q, hq, _ = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    lo, hi = block * b, min(block * (b + 1), n_k)
    dki = np.zeros((max(hi - lo, 0), q_idx.shape[2]))
    for i in range(n_q):
        if not np.any(sel[i, g] == b):
            continue
        keys = _key_set(sel[i, g], n_k, block, int(pos[i]), causal)
        mine = (keys >= lo) & (keys < hi)
        if not mine.any():
            continue
        dz, _ = _row_terms(q, k, q_idx, k_idx, keys, i, g, grp, scale, proxy_scale)
        dki[keys[mine] - lo] += np.outer(dz[mine], q_idx[i, g])
    return dki
