"""Plain fp64 CPU oracle of the per-Q-tile block selectors R1 and R4.

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code with the HIP path.

"Sparse Attention", Chapter 4 (R1: one representative; R4: four representatives): each
128-query tile and each 128-key block is summarised by the average of its token vectors
(R1), or by the averages of its four consecutive 32-token groups (R4), per head. A block's
score for a (tile, GQA group) is the largest dot product between a query representative of
any query head of the group and a key representative of the block; each tile and group
keeps the 16 (here: topk) best blocks.

Readings where the chapter is silent: the representatives average the token values as
stored (no softmax scale; a positive scale cannot change the selection); a ragged last tile
or block averages the tokens it has, and a representative group with no token takes part
in no comparison; ties go to the lower block index and lists are ordered by score
descending, then block index; with causal masking a block is visible to a tile when its
first key is not after the position of the tile's last query (bottom-right aligned), and no
block is forced; fewer visible blocks than topk leave -1 slots.
"""
from __future__ import annotations

import numpy as np

from oracle.msa_ref import NEG_INF, n_blocks, query_positions, select_topk


def representatives(x: np.ndarray, reps: int, block: int) -> np.ndarray:
    """x [T, H, D] (fp64) -> [ceil(T / block), H, reps, D]: the mean of each of the `reps`
    consecutive groups of block / reps tokens of every block; NaN for a group with no token."""
    t, h, d = x.shape
    nb = n_blocks(t, block)
    size = block // reps
    out = np.full((nb, h, reps, d), np.nan)
    for b in range(nb):
        for r in range(reps):
            lo = b * block + r * size
            hi = min(lo + size, t)
            if lo < hi:
                out[b, :, r, :] = x[lo:hi].mean(axis=0)
    return out


def tile_block_scores(q: np.ndarray, k: np.ndarray, reps: int, block: int, group: int,
                      causal: bool) -> np.ndarray:
    """Scores [tiles, Hkv, nb] of one sequence: q [N, Hq, D], k [Nk, Hkv, D] (fp64)."""
    n_q, n_k = q.shape[0], k.shape[0]
    qr = representatives(q, reps, block)           # [tiles, Hq, R, D]
    kr = representatives(k, reps, block)           # [nb, Hkv, R, D]
    tiles, nb, hkv = qr.shape[0], kr.shape[0], k.shape[1]
    out = np.full((tiles, hkv, nb), NEG_INF)
    pos = query_positions(n_q, n_k)
    for t in range(tiles):
        last = pos[min((t + 1) * block, n_q) - 1]
        for g in range(hkv):
            qv = qr[t, g * group:(g + 1) * group].reshape(group * reps, -1)
            for b in range(nb):
                if causal and b * block > last:
                    continue
                kv = kr[b, g]
                dots = qv @ kv.T                    # NaN where either group is empty
                if np.any(~np.isnan(dots)):
                    out[t, g, b] = np.nanmax(dots)
    return out


def select_tiles(q: np.ndarray, k: np.ndarray, reps: int, block: int, group: int, topk: int,
                 causal: bool) -> tuple[np.ndarray, np.ndarray]:
    """Per-tile lists [tiles, Hkv, topk] int32 (score descending, block ascending, -1 padding)
    and the scores [tiles, Hkv, nb] of one sequence."""
    s = tile_block_scores(q, k, reps, block, group, causal)
    return select_topk(s, topk), s
