"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test fixes the oracle against a library routine, a brute-force or alternative
algorithm, an invariant, a closed form, or a value the pages print. The planted-mistake
tests at the end alter the oracle in plausible ways and check that some pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import msa_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, k, v, mask, scale):
    """torch's scaled_dot_product_attention on CPU in float64; q [N, Hq, D], k/v [Nk, Hkv, D],
    mask [N, Nk] bool (True = attend) shared by all heads; GQA by repeating K/V heads."""
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    m = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def bottom_right_causal(n_q, n_k):
    i = np.arange(n_q)[:, None]
    u = np.arange(n_k)[None, :]
    return u <= (n_k - n_q) + i


def all_blocks_lists(n_q, hkv, nb):
    return np.broadcast_to(np.arange(nb, dtype=np.int32), (n_q, hkv, nb)).copy()


# ------------------------------------------------------------------ special cases vs SDPA

@pytest.mark.parametrize("n_q,n_k", [(512, 512), (200, 512), (384, 300)])
def test_dense_special_case_causal_matches_sdpa(n_q, n_k):
    """With K >= number of blocks every visible block is selected, so the sparse layer is
    plain causal attention (bottom-right aligned)."""
    hq, hkv, d, dp, blk = 6, 2, 16, 8, 128
    q, k, v = rnd(1, n_q, hq, d), rnd(2, n_k, hkv, d), rnd(3, n_k, hkv, d)
    qi, ki = rnd(4, n_q, hkv, dp), rnd(5, n_k, hkv, dp)
    nb = ref.n_blocks(n_k, blk)
    sel, _ = ref.index_topk(qi, ki, blk, nb + 1, causal=True)
    o, lse = ref.sparse_attention(q, k, v, sel, 0.25, blk, causal=True)
    mask = bottom_right_causal(n_q, n_k)
    has_key = mask.any(axis=1)
    expect = sdpa(q, k, v, mask | ~has_key[:, None], 0.25)
    np.testing.assert_allclose(o[has_key], expect[has_key], rtol=0, atol=1e-12)
    assert np.all(o[~has_key] == 0) and np.all(np.isneginf(lse[~has_key]))
    # LSE against scipy's logsumexp of the masked scores
    x = 0.25 * np.einsum("ihd,uhd->ihu", q, np.repeat(k, hq // hkv, axis=1))
    x = np.where(mask[:, None, :], x, -np.inf)
    np.testing.assert_allclose(lse[has_key], logsumexp(x, axis=2)[has_key], atol=1e-12)


def test_dense_special_case_noncausal_matches_sdpa():
    n_q, n_k, hq, hkv, d, blk = 130, 333, 4, 4, 8, 128
    q, k, v = rnd(11, n_q, hq, d), rnd(12, n_k, hkv, d), rnd(13, n_k, hkv, d)
    nb = ref.n_blocks(n_k, blk)
    sel = all_blocks_lists(n_q, hkv, nb)
    o, _ = ref.sparse_attention(q, k, v, sel, 0.3, blk, causal=False)
    expect = sdpa(q, k, v, np.ones((n_q, n_k), bool), 0.3)
    np.testing.assert_allclose(o, expect, atol=1e-12)


def test_local_only_special_case_matches_block_diagonal_sdpa():
    """With K = 1 only the forced local block survives: block-diagonal causal attention."""
    n, hq, hkv, d, dp, blk = 512, 4, 1, 16, 8, 128
    q, k, v = rnd(21, n, hq, d), rnd(22, n, hkv, d), rnd(23, n, hkv, d)
    qi, ki = rnd(24, n, hkv, dp), rnd(25, n, hkv, dp)
    sel, _ = ref.index_topk(qi, ki, blk, 1, causal=True)
    assert np.all(sel[:, 0, 0] == np.arange(n) // blk)
    o, _ = ref.sparse_attention(q, k, v, sel, 1 / math.sqrt(d), blk, causal=True)
    i = np.arange(n)[:, None]
    u = np.arange(n)[None, :]
    mask = (u <= i) & (u // blk == i // blk)
    np.testing.assert_allclose(o, sdpa(q, k, v, mask, 1 / math.sqrt(d)), atol=1e-12)


def test_worked_list_example_from_pages():
    """'Sparse Attention', Chapter 2: list [2, 5, 8] with count 3 visits KV2, KV5, KV8."""
    g = json.load(open(os.path.join(GOLDEN, "sparse_attention_worked_example.json")))
    blk = g["block"]
    n_q, n_k, hq, hkv, d = 128, 10 * blk, 2, 1, 16
    q, k, v = rnd(31, n_q, hq, d), rnd(32, n_k, hkv, d), rnd(33, n_k, hkv, d)
    lst = np.full((1, hkv, 4), -1, dtype=np.int32)          # one Q tile, -1 after the count
    lst[0, 0, :g["selected_count"]] = g["selected_indices"]
    sel = ref.lists_for_queries(lst, n_q, 128)
    o, _ = ref.sparse_attention(q, k, v, sel, 0.2, blk, causal=False)
    keys = np.concatenate([np.arange(b * blk, (b + 1) * blk) for b in g["visited_blocks"]])
    expect = sdpa(q, k[keys], v[keys], np.ones((n_q, keys.size), bool), 0.2)
    np.testing.assert_allclose(o, expect, atol=1e-12)


# ------------------------------------------------------------------ selection, brute force

def exact_scores(qi, ki, blk, causal, rows=None):
    """Exact (Python integer) max-pooled block scores for integer-valued proxies, by explicit
    loops over keys; None for a block with no visible key. Returns {row: [[score per block]
    per group]}."""
    n_q, hkv, dp = qi.shape
    n_k = ki.shape[0]
    nb = -(-n_k // blk)
    qint = qi.astype(np.int64).tolist()
    kint = ki.astype(np.int64).tolist()
    out = {}
    for i in (range(n_q) if rows is None else rows):
        i = int(i)
        pos = n_k - n_q + i
        per_g = []
        for g in range(hkv):
            qv = qint[i][g]
            row = []
            for j in range(nb):
                best = None
                for u in range(j * blk, min(n_k, (j + 1) * blk)):
                    if causal and u > pos:
                        break
                    s = sum(a * b for a, b in zip(qv, kint[u][g]))
                    best = s if best is None or s > best else best
                row.append(best)
            per_g.append(row)
        out[i] = per_g
    return out


def brute_select(scores_row, local, topk):
    """Sorted() on (-score, index) over visible non-local blocks, local block first."""
    cand = [(-s, j) for j, s in enumerate(scores_row) if s is not None and j != local]
    chosen = [j for _, j in sorted(cand)]
    lst = ([local] if local is not None else []) + chosen
    lst = lst[:topk]
    return lst + [-1] * (topk - len(lst))


def streaming_insertion(scores_row, local, topk):
    """The proxy page's method: blocks arrive in ascending order, each block max is inserted
    into a running top list kept sorted, a new value going after equal ones."""
    vals, ids = [], []
    for j, s in enumerate(scores_row):
        if s is None or j == local:
            continue
        p = len(vals)
        while p > 0 and vals[p - 1] < s:
            p -= 1
        vals.insert(p, s)
        ids.insert(p, j)
        del vals[topk - 1:], ids[topk - 1:]
    lst = ([local] if local is not None else []) + ids
    lst = lst[:topk]
    return lst + [-1] * (topk - len(lst))


@pytest.mark.parametrize("n_q,n_k,hkv,dp,topk,causal", [
    (256, 640, 1, 4, 2, True), (384, 384, 2, 4, 3, True), (130, 512, 1, 8, 3, True),
    (200, 450, 2, 4, 3, False),
])
def test_selection_matches_exact_brute_force(n_q, n_k, hkv, dp, topk, causal):
    """Small-integer proxies: exact rational dot products, many ties."""
    blk = 128
    rng = np.random.default_rng(n_q + n_k + dp)
    qi = rng.integers(-2, 3, size=(n_q, hkv, dp)).astype(np.float64)
    ki = rng.integers(-2, 3, size=(n_k, hkv, dp)).astype(np.float64)
    # thin out rows so that the test stays fast: all blocks, a spread of queries
    rows = np.unique(np.concatenate([np.arange(0, n_q, 7), [n_q - 1]]))
    sel, _ = ref.index_topk(qi, ki, blk, topk, causal, rows=rows)
    ex = exact_scores(qi, ki, blk, causal, rows)
    n_tie = 0
    for ri, i in enumerate(rows):
        pos = n_k - n_q + i
        loc = pos // blk if 0 <= pos // blk < -(-n_k // blk) else None
        for g in range(hkv):
            row = ex[i][g]
            bf = brute_select(row, loc, topk)
            st = streaming_insertion(row, loc, topk)
            assert bf == st
            assert list(sel[ri, g]) == bf, (i, g, row)
            vis = [s for j, s in enumerate(row) if s is not None and j != loc]
            n_tie += len(vis) - len(set(vis))
    assert n_tie > 0, "inputs should exercise the tie rule"


def test_selection_properties_on_gaussian_proxies():
    n, hkv, dp, blk, topk = 1024, 2, 16, 128, 4
    qi, ki = rnd(41, n, hkv, dp), rnd(42, n, hkv, dp)
    sel, sc = ref.index_topk(qi, ki, blk, topk, causal=True)
    for i in range(n):
        c = i // blk
        for g in range(hkv):
            lst = [b for b in sel[i, g] if b >= 0]
            assert sel[i, g, 0] == c                          # local block, slot 0
            assert len(lst) == min(topk, c + 1)               # count
            assert len(set(lst)) == len(lst)                  # distinct
            assert all(0 <= b <= c for b in lst)              # visible
            chosen = set(lst[1:])
            worst = min([sc[i, g, b] for b in chosen], default=np.inf)
            rest = [sc[i, g, b] for b in range(c) if b not in chosen]
            assert all(r <= worst for r in rest)
            # slots after the local one are score-descending
            vals = [sc[i, g, b] for b in lst[1:]]
            assert vals == sorted(vals, reverse=True)


# ------------------------------------------------------------------ invariants

def test_constant_values_give_constant_output_and_weights_sum_to_one():
    n, hq, hkv, d, dp, blk, topk = 640, 4, 2, 8, 8, 128, 3
    q, k = rnd(51, n, hq, d), rnd(52, n, hkv, d)
    qi, ki = rnd(53, n, hkv, dp), rnd(54, n, hkv, dp)
    sel, _ = ref.index_topk(qi, ki, blk, topk, causal=True)
    o, _ = ref.sparse_attention(q, k, np.ones((n, hkv, d)), sel, 0.3, blk, causal=True)
    np.testing.assert_allclose(o, 1.0, atol=1e-13)


def test_one_hot_values_expose_weights_support_and_sum():
    """V[u] = e_u makes O[i, h, u] the weight on key u: it must be positive exactly on the
    causally visible keys of the selected blocks, and the weights must sum to one."""
    n, hq, hkv, dp, blk, topk = 512, 2, 1, 8, 128, 2
    q, k = rnd(61, n, hq, 16), rnd(62, n, hkv, 16)
    qi, ki = rnd(63, n, hkv, dp), rnd(64, n, hkv, dp)
    v = np.eye(n)[:, None, :]                                     # D = n
    sel, _ = ref.index_topk(qi, ki, blk, topk, causal=True)
    o, lse = ref.sparse_attention(q, k, v, sel, 0.25, blk, causal=True)
    u = np.arange(n)
    for i in range(0, n, 5):
        allowed = np.isin(u // blk, sel[i, 0]) & (u <= i)
        for h in range(hq):
            assert np.all(o[i, h, ~allowed] == 0)
            assert np.all(o[i, h, allowed] > 0)
            assert abs(o[i, h].sum() - 1.0) < 1e-12
            x = 0.25 * (k[allowed, 0] @ q[i, h])
            assert lse[i, h] >= x.max() - 1e-12
            assert lse[i, h] <= x.max() + math.log(allowed.sum()) + 1e-12


# ------------------------------------------------------------------ partials and combine

def test_combine_identity_and_scipy_softmax():
    n, hq, hkv, d, dp, blk, topk = 700, 4, 2, 8, 8, 128, 4
    q, k, v = rnd(71, n, hq, d), rnd(72, n, hkv, d), rnd(73, n, hkv, d)
    qi, ki = rnd(74, n, hkv, dp), rnd(75, n, hkv, dp)
    sel, _ = ref.index_topk(qi, ki, blk, topk, causal=True)
    o_s, l_s = ref.partial_attention(q, k, v, sel, 0.2, blk, causal=True)
    o_c, l_c = ref.combine(o_s, l_s)
    o, l = ref.sparse_attention(q, k, v, sel, 0.2, blk, causal=True)
    np.testing.assert_allclose(o_c, o, atol=1e-12)
    np.testing.assert_allclose(l_c, l, atol=1e-12)
    # the merge is softmax(lse) over slots, checked with scipy on rows with finite slots
    i = 500
    lw = l_s[i, 0]
    fin = np.isfinite(lw)
    w = softmax(lw[fin])
    np.testing.assert_allclose(o_c[i, 0], (w[:, None] * o_s[i, 0][fin]).sum(0), atol=1e-12)
    np.testing.assert_allclose(l_c[i, 0], logsumexp(lw[fin]), atol=1e-12)


def test_union_semantics_duplicates_invalid_and_permutation():
    n, hq, hkv, d, blk = 256, 2, 1, 8, 128
    n_k = 1000
    q, k, v = rnd(81, n, hq, d), rnd(82, n_k, hkv, d), rnd(83, n_k, hkv, d)
    base = np.array([3, 0, 7, 5], dtype=np.int32)
    sel = np.broadcast_to(base, (n, hkv, 4)).copy()
    o1, l1 = ref.sparse_attention(q, k, v, sel, 0.2, blk, causal=False)
    perm = sel[:, :, ::-1].copy()
    o2, l2 = ref.sparse_attention(q, k, v, perm, 0.2, blk, causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    dup = np.broadcast_to(np.array([3, 0, 3, 7, 5, -1, 99, 5], np.int32), (n, hkv, 8)).copy()
    o3, l3 = ref.sparse_attention(q, k, v, dup, 0.2, blk, causal=False)
    np.testing.assert_allclose(o1, o3, atol=1e-12)
    o_s, l_s = ref.partial_attention(q, k, v, dup, 0.2, blk, causal=False)
    o4, l4 = ref.combine(o_s, l_s)
    np.testing.assert_allclose(o4, o1, atol=1e-12)
    np.testing.assert_allclose(l4, l1, atol=1e-12)
    # last block (7) holds only 1000 - 896 = 104 keys
    keys = np.concatenate([np.arange(b * blk, min(n_k, (b + 1) * blk)) for b in (0, 3, 5, 7)])
    np.testing.assert_allclose(o1, sdpa(q, k[keys], v[keys], np.ones((n, keys.size), bool), 0.2),
                               atol=1e-12)


def test_empty_rows():
    """A query whose lists hold no visible key: O = 0, LSE = -inf, also through combine."""
    n, hq, hkv, d, blk = 128, 2, 1, 4, 128
    q, k, v = rnd(91, n, hq, d), rnd(92, 512, hkv, d), rnd(93, 512, hkv, d)
    sel = np.full((n, hkv, 2), -1, dtype=np.int32)
    o, l = ref.sparse_attention(q, k, v, sel, 0.2, blk, causal=True)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    o_s, l_s = ref.partial_attention(q, k, v, sel, 0.2, blk, causal=True)
    o2, l2 = ref.combine(o_s, l_s)
    assert np.all(o2 == 0) and np.all(np.isneginf(l2))


# ------------------------------------------------------------------ input rounding

def e4m3fn_values():
    """All finite OCP e4m3fn values from the format's definition: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits, subnormals at exponent 0, code 0x7F/0xFF is NaN, no inf."""
    vals = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((-mag if s else mag, code))
    return vals


def test_fp8_input_rounding_is_rne_with_saturation():
    from synth.msa_inputs import to_fp8
    table = sorted({v for v, _ in e4m3fn_values()})
    pos = np.array([v for v in table if v >= 0])
    assert pos.max() == 448.0
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 3, pos[:-1] + np.diff(pos) / 2, [-7.0, 0.0]])
    x = x.astype(np.float32)
    t, scale = to_fp8(x)
    got = t.to(torch.float64).numpy()
    y = np.clip(x.astype(np.float64) / scale, -448, 448)
    # nearest table value, ties to the even code (lowest mantissa bit 0)
    codes = {v: c for v, c in e4m3fn_values()}
    for xi, gi in zip(y, got):
        a = abs(xi)
        j = np.searchsorted(pos, a)
        cands = [pos[max(0, j - 1)], pos[min(len(pos) - 1, j)]]
        dists = [abs(c - a) for c in cands]
        if dists[0] == dists[1] and cands[0] != cands[1]:
            best = cands[0] if codes[cands[0]] % 2 == 0 else cands[1]
        else:
            best = cands[int(np.argmin(dists))]
        assert abs(gi) == best and (gi == 0 or np.sign(gi) == np.sign(xi)), (xi, gi, best)


def test_bf16_input_rounding_is_rne():
    from synth.msa_inputs import to_bf16
    rng = np.random.default_rng(6)
    x = rng.standard_normal(50000).astype(np.float32)
    bits = x.view(np.uint32)
    # ties: low 16 bits exactly 0x8000
    ties = ((bits[:1000] & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    got = to_bf16(x).view(torch.int16).numpy().astype(np.uint16)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    want = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ planted mistakes

def _dense_case():
    n_q, n_k, hq, hkv, d, dp, blk = 200, 512, 4, 2, 8, 8, 128
    return (rnd(101, n_q, hq, d), rnd(102, n_k, hkv, d), rnd(103, n_k, hkv, d),
            rnd(104, n_q, hkv, dp), rnd(105, n_k, hkv, dp), blk)


def _dense_pin_passes():
    q, k, v, qi, ki, blk = _dense_case()
    nb = ref.n_blocks(k.shape[0], blk)
    sel, _ = ref.index_topk(qi, ki, blk, nb, causal=True)
    o, _ = ref.sparse_attention(q, k, v, sel, 0.3, blk, causal=True)
    return np.allclose(o, sdpa(q, k, v, bottom_right_causal(q.shape[0], k.shape[0]), 0.3),
                       atol=1e-10)


def _tie_pin_passes():
    rng = np.random.default_rng(7)
    qi = rng.integers(-1, 2, size=(640, 1, 2)).astype(np.float64)
    ki = rng.integers(-1, 2, size=(640, 1, 2)).astype(np.float64)
    rows = range(256, 640, 3)
    sel, _ = ref.index_topk(qi, ki, 128, 3, True)
    ex = exact_scores(qi, ki, 128, True, rows)
    return all(list(sel[i, 0]) == brute_select(ex[i][0], i // 128, 3) for i in rows)


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _dense_pin_passes() and _tie_pin_passes()
    # top-left instead of bottom-right causal alignment
    with monkeypatch.context() as m:
        m.setattr(ref, "query_positions", lambda n_q, n_k: np.arange(n_q, dtype=np.int64))
        assert not _dense_pin_passes()
    # ties broken toward the higher block index
    orig = ref.select_topk

    def tie_high(scores, topk):
        flipped = scores[:, :, ::-1]
        s = orig(flipped, topk)
        nb = scores.shape[2]
        return np.where(s >= 0, nb - 1 - s, -1).astype(np.int32)
    with monkeypatch.context() as m:
        m.setattr(ref, "select_topk", tie_high)
        assert not _tie_pin_passes()
    # softmax scale dropped
    orig_attend = ref.attend
    with monkeypatch.context() as m:
        m.setattr(ref, "attend", lambda qh, kk, vv, scale: orig_attend(qh, kk, vv, 1.0))
        assert not _dense_pin_passes()
    # keys of the local block past the query's position left visible
    orig_keys = ref._key_set
    with monkeypatch.context() as m:
        m.setattr(ref, "_key_set", lambda b, n_k, blk, pos, causal: orig_keys(b, n_k, blk, pos, False))
        assert not _dense_pin_passes()
