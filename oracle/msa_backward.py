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
