"""Plain fp64 CPU oracle of the main-branch backward of block-sparse GQA attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path.

"Flash-MSA: accelerating million-token training" keeps the selected block ids and the main
branch's log-sum-exp for the backward; the gradients are those of exact softmax attention
restricted to each query's union of selected keys (the forward definition of
"Kernel optimization for MiniMax M3 on NVIDIA Blackwell", summary). Per query row i, head h
(group g), key set S(i, g) and scale tau, with P_iu = exp(tau q_i . k_u - LSE_i):

    dV_u  += sum_(i, h in g) P_iu dO_i
    dP_iu  = dO_i . v_u
    D_i    = dO_i . O_i                      (= sum_u P_iu dP_iu)
    dS_iu  = P_iu (dP_iu - D_i)
    dQ_i   = tau sum_u dS_iu k_u
    dK_u  += tau sum_(i, h in g) dS_iu q_i

The selection itself (the index branch) is not differentiated: the lists are inputs.
"""
from __future__ import annotations

import numpy as np

from oracle.msa_ref import _key_set, attend, query_positions


def sparse_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
                              do: np.ndarray, scale: float, block: int, causal: bool
                              ) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray,
                                         np.ndarray]:
    """One sequence: q [N, Hq, D], k / v [Nk, Hkv, D], sel [N, Hkv, K], dO [N, Hq, D] (fp64).
    Returns (dQ [N, Hq, D], dK [Nk, Hkv, D], dV [Nk, Hkv, D], O [N, Hq, D], LSE [N, Hq]).
    A row with no visible key has O = 0, LSE = -inf and contributes nothing."""
    n_q, hq, d = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((n_q, hq), -np.inf)
    for i in range(n_q):
        for g in range(hkv):
            keys = _key_set(sel[i, g], n_k, block, int(pos[i]), causal)
            if keys.size == 0:
                continue
            heads = slice(g * grp, (g + 1) * grp)
            kk, vv = k[keys, g], v[keys, g]
            oi, li = attend(q[i, heads], kk, vv, scale)
            o[i, heads], lse[i, heads] = oi, li
            p = np.exp(scale * (q[i, heads] @ kk.T) - li[:, None])      # [G, S]
            dpi = do[i, heads] @ vv.T                                   # [G, S]
            di = np.sum(do[i, heads] * oi, axis=1, keepdims=True)       # [G, 1]
            ds = p * (dpi - di)
            dq[i, heads] = scale * (ds @ kk)
            np.add.at(dk[:, g], keys, scale * (ds.T @ q[i, heads]))
            np.add.at(dv[:, g], keys, p.T @ do[i, heads])
    return dq, dk, dv, o, lse


def run_case(case, dout, lists: np.ndarray | None = None):
    """The backward of a whole seeded case: per sequence, on the lists the oracle's own index
    branch selects (or the case's per-tile lists, or ``lists`` [Tq, Hkv, K] when given).
    Returns (dQ [Tq, Hq, D], dK, dV [Tk, Hkv, D], O, LSE, per-query lists [Tq, Hkv, K])."""
    from oracle import msa_case
    from synth.msa_inputs import widen
    cfg = case.cfg
    dsq, dsk, dsv = case.descale
    q, k, v = widen(case.q, dsq), widen(case.k, dsk), widen(case.v, dsv)
    g_out = widen(dout)
    if lists is None:
        lists = np.full((case.total_q, cfg.hkv, cfg.topk), -1, dtype=np.int32)
        sel = msa_case.run(case, want_output=False)
        if sel.rows is not None:
            lists[sel.rows] = sel.topk_idx
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.full((case.total_q, cfg.hq), -np.inf)
    for s in range(len(case.cu_q) - 1):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        k0, k1 = int(case.cu_k[s]), int(case.cu_k[s + 1])
        if q1 == q0:
            continue
        r = sparse_attention_backward(q[q0:q1], k[k0:k1], v[k0:k1], lists[q0:q1], g_out[q0:q1],
                                      case.softmax_scale, cfg.block, cfg.causal)
        dq[q0:q1], dk[k0:k1], dv[k0:k1], o[q0:q1], lse[q0:q1] = r
    return dq, dk, dv, o, lse, lists


def query_rows_gradient(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel_rows: np.ndarray,
                        do_rows: np.ndarray, rows: np.ndarray, scale: float, block: int,
                        causal: bool) -> np.ndarray:
    """dQ of the given query ``rows`` of one sequence only (each row's dQ depends on its own
    list, O and LSE alone): q [N, Hq, D], k / v [Nk, Hkv, D], sel_rows [R, Hkv, K], do_rows
    [R, Hq, D]; the same formulas as sparse_attention_backward. Returns [R, Hq, D]."""
    n_q, hq, _ = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    out = np.zeros((rows.size, hq, q.shape[2]))
    for r, i in enumerate(rows):
        for g in range(hkv):
            keys = _key_set(sel_rows[r, g], n_k, block, int(pos[i]), causal)
            if keys.size == 0:
                continue
            heads = slice(g * grp, (g + 1) * grp)
            kk, vv = k[keys, g], v[keys, g]
            oi, li = attend(q[i, heads], kk, vv, scale)
            p = np.exp(scale * (q[i, heads] @ kk.T) - li[:, None])
            ds = p * (do_rows[r, heads] @ vv.T - np.sum(do_rows[r, heads] * oi, axis=1,
                                                         keepdims=True))
            out[r, heads] = scale * (ds @ kk)
    return out


def key_block_gradient(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
                       do: np.ndarray, g: int, b: int, scale: float, block: int, causal: bool
                       ) -> tuple[np.ndarray, np.ndarray]:
    """dK and dV of the keys of block ``b`` of group ``g`` only (one (group, block) column):
    the sum, over the queries whose list for g holds b, of their terms in the formulas of
    sparse_attention_backward, each query's P and D taken over its own whole key set.
    q [N, Hq, D], k / v [Nk, Hkv, D], sel [N, Hkv, K], do [N, Hq, D] (fp64).
    Returns (dK, dV), each [n_b, D] for the keys block*b .. min(block*(b+1), Nk) - 1."""
    n_q, hq, d = q.shape
    n_k, hkv, _ = k.shape
    grp = hq // hkv
    pos = query_positions(n_q, n_k)
    lo, hi = block * b, min(block * (b + 1), n_k)
    dk = np.zeros((max(hi - lo, 0), d))
    dv = np.zeros((max(hi - lo, 0), d))
    heads = slice(g * grp, (g + 1) * grp)
    for i in range(n_q):
        if not np.any(sel[i, g] == b):
            continue
        keys = _key_set(sel[i, g], n_k, block, int(pos[i]), causal)
        mine = (keys >= lo) & (keys < hi)
        if not mine.any():
            continue
        kk, vv = k[keys, g], v[keys, g]
        oi, li = attend(q[i, heads], kk, vv, scale)
        p = np.exp(scale * (q[i, heads] @ kk.T) - li[:, None])          # [G, S]
        ds = p * (do[i, heads] @ vv.T - np.sum(do[i, heads] * oi, axis=1, keepdims=True))
        at = keys[mine] - lo
        dk[at] += scale * (ds[:, mine].T @ q[i, heads])
        dv[at] += p[:, mine].T @ do[i, heads]
    return dk, dv
