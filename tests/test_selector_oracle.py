"""Pins of the per-Q-tile selector oracle (R1, R4: "Sparse Attention", Chapter 4) against a
closed form and exact brute force."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import selectors as S


def _brute(q, k, reps, block, group, topk, causal):
    """Exact rational means and dots on integer inputs, then a full sort by (-score, block)."""
    n_q, hq, d = q.shape
    n_k, hkv, _ = k.shape
    size = block // reps

    def reps_of(x, t0, h):
        out = []
        for r in range(reps):
            lo, hi = t0 + r * size, min(t0 + (r + 1) * size, x.shape[0])
            if lo < hi:
                out.append([Fraction(int(sum(int(x[u, h, e]) for u in range(lo, hi))), hi - lo)
                            for e in range(d)])
        return out

    tiles, nb = -(-n_q // block), -(-n_k // block)
    lists = np.full((tiles, hkv, topk), -1, dtype=np.int64)
    scores = {}
    for t in range(tiles):
        last = n_k - n_q + min((t + 1) * block, n_q) - 1
        for g in range(hkv):
            cand = []
            for b in range(nb):
                if causal and b * block > last:
                    continue
                best = None
                for h in range(g * group, (g + 1) * group):
                    for qv in reps_of(q, t * block, h):
                        for kv in reps_of(k, b * block, g):
                            s = sum(a * c for a, c in zip(qv, kv))
                            best = s if best is None or s > best else best
                if best is not None:
                    cand.append((-best, b))
                    scores[(t, g, b)] = best
            cand.sort()
            for i, (_, b) in enumerate(cand[:topk]):
                lists[t, g, i] = b
    return lists, scores


@pytest.mark.parametrize("reps", [1, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_selectors_match_exact_brute_force(reps, causal):
    rng = np.random.default_rng(11 + reps + 2 * causal)
    # ragged: the last tile holds 72 queries (groups of 32, 32, 8 and none), the last block
    # 44 keys (32, 12, none, none)
    q = rng.integers(-3, 4, size=(200, 4, 4)).astype(np.float64)
    k = rng.integers(-3, 4, size=(300, 2, 4)).astype(np.float64)
    lists, sc = S.select_tiles(q, k, reps, 128, 2, 2, causal)
    want, wsc = _brute(q, k, reps, 128, 2, 2, causal)
    assert np.array_equal(lists, want)
    for (t, g, b), v in wsc.items():
        assert abs(sc[t, g, b] - float(v)) <= 1e-12 * max(1.0, abs(float(v)))
    assert np.sum(np.isfinite(sc)) == len(wsc)


@pytest.mark.parametrize("reps", [1, 4])
def test_block_constant_inputs_reduce_to_a_matrix_product(reps):
    """Tokens constant within each tile (per head) and within each block: every
    representative is that constant, so the scores are max over the group's heads of a . c."""
    rng = np.random.default_rng(3)
    tiles, nb, hq, hkv, d, g = 3, 5, 8, 2, 16, 4
    a = rng.standard_normal((tiles, hq, d))
    c = rng.standard_normal((nb, hkv, d))
    q = np.repeat(a, 128, axis=0)
    k = np.repeat(c, 128, axis=0)
    lists, sc = S.select_tiles(q, k, reps, 128, g, 4, False)
    want = np.stack([np.einsum("thd,bd->thb", a[:, gg * g:(gg + 1) * g], c[:, gg]).max(axis=1)
                     for gg in range(hkv)], axis=1)                 # [tiles, hkv, nb]
    np.testing.assert_allclose(sc, want, rtol=1e-12, atol=1e-12)
    order = np.argsort(-want, axis=2, kind="stable")[:, :, :4]
    assert np.array_equal(lists, order)


def test_r4_ignores_order_inside_each_32_token_group_and_r1_inside_each_block():
    rng = np.random.default_rng(5)
    q = rng.integers(-4, 5, size=(256, 2, 8)).astype(np.float64)
    k = rng.integers(-4, 5, size=(512, 1, 8)).astype(np.float64)
    base4 = S.select_tiles(q, k, 4, 128, 2, 3, False)
    base1 = S.select_tiles(q, k, 1, 128, 2, 3, False)
    perm32 = np.concatenate([rng.permutation(32) + 32 * i for i in range(16)])
    q4, k4 = q[perm32[:256]], k[perm32]
    got4 = S.select_tiles(q4, k4, 4, 128, 2, 3, False)
    assert np.array_equal(got4[0], base4[0]) and np.array_equal(got4[1], base4[1])
    perm128 = np.concatenate([rng.permutation(128) + 128 * i for i in range(4)])
    got1 = S.select_tiles(q[perm128[:256]], k[perm128], 1, 128, 2, 3, False)
    assert np.array_equal(got1[0], base1[0]) and np.array_equal(got1[1], base1[1])
    # a key moved across a 32-token group boundary inside its block: R1 is blind to it, R4 not
    k2 = k.copy()
    k2[[5, 40]] = k2[[40, 5]]
    assert np.array_equal(S.select_tiles(q, k2, 1, 128, 2, 3, False)[1], base1[1])
    assert not np.array_equal(S.select_tiles(q, k2, 4, 128, 2, 3, False)[1], base4[1])
