"""GPU path (libmsa through its C ABI) against the fp64 oracle on seeded inputs.

Bars: block lists bit-exact (grid-valued proxies make every fp32 dot product exact; on
Gaussian proxies a differing list is accepted only as a certified near-tie, and its rows are
left out of the output comparison); outputs max |O - O_ref| <= 2e-2 for bf16 and 6e-2 for
fp8; |LSE - LSE_ref| <= 1e-2 (bf16) / 5e-2 (fp8); partial outputs and LSEs against the
oracle's per-slot partials at the same bars.
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case, msa_ref as ref
from synth import msa_inputs as mi
from synth.msa_inputs import widen

from gpu_util import (compare_lists, err_stats, gpu_attention, gpu_index, proxies,
                      proxy_score_errors, shape_of, upload)

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "fp8": (6e-2, 5e-2)}


def _say(*a):
    print(*a, flush=True)


def _oracle_index_scores(case):
    """Per-sequence fp64 block scores of the oracle, addressed by global row."""
    out = msa_case.run(case, want_output=False)
    seq_of = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1

    def scores(i, g):
        s = seq_of[i]
        return out.scores[s][i - case.cu_q[s], g]
    return out, scores


def _err_fn(case):
    """(row, group) -> per-block error bounds of the computed proxy scores (fp64)."""
    qi, ki = proxies(case)
    seq_of = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1

    def err(i, g):
        s = seq_of[i]
        k0, k1 = case.cu_k[s], case.cu_k[s + 1]
        pos = (k1 - k0) - (case.cu_q[s + 1] - case.cu_q[s]) + (i - case.cu_q[s])
        return proxy_score_errors(qi[i, g], ki[k0:k1, g], int(pos) if case.cfg.causal else None,
                                  case.cfg.idx_dtype == "fp8")
    return err


# ------------------------------------------------------------------ index branch

INDEX_CASES = [
    ("tiny_grid", dict(n_q=(2048,), hq=16, hkv=1, topk=4, dp=32, proxy="grid")),
    ("ragged_varlen_grid", dict(n_q=(300, 1, 640, 129), n_k=(700, 4000, 640, 129), hq=8, hkv=2,
                                topk=5, dp=64, proxy="grid")),
    ("noncausal_grid", dict(n_q=(200, 384), n_k=(1000, 384), hq=4, hkv=2, topk=6, dp=32,
                            causal=False, proxy="grid")),
    ("decode_grid", dict(n_q=(1, 1, 1, 2), n_k=(130, 4096 + 77, 9000, 256), hq=16, hkv=2,
                         topk=16, dp=64, proxy="grid")),
    # short-query (key-split) path: one, three and eight groups, non-causal rows, and more
    # than 64 key chunks per query
    ("split_g1", dict(n_q=(1, 3), n_k=(5000, 20000), hq=4, hkv=1, topk=16, dp=32, proxy="grid")),
    ("split_g3", dict(n_q=(2,), n_k=(9000,), hq=6, hkv=3, topk=8, dp=64, proxy="grid")),
    ("split_g8", dict(n_q=(1, 1), n_k=(3000, 12000), hq=16, hkv=8, topk=16, dp=64, proxy="grid")),
    ("split_noncausal", dict(n_q=(4, 16), n_k=(3000, 7000), hq=8, hkv=4, topk=10, dp=32,
                             causal=False, proxy="grid")),
    ("split_many_chunks", dict(n_q=(1,), n_k=(300000,), hq=2, hkv=1, topk=16, dp=32,
                               proxy="grid")),
]


@pytest.mark.parametrize("name,kw", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_topk_bit_exact_on_exact_arithmetic(name, kw):
    _say(f"[index exact] {name}")
    case = mi.make_case(mi.custom(name=name, **kw), seed=1)
    got, got_sc = gpu_index(case, upload(case))
    out = msa_case.run(case, want_output=False)
    n_diff, _, bad = compare_lists(got, out.topk_idx, None)
    assert n_diff == 0, f"{n_diff} rows differ, first {bad[:5]}"
    # scores of the selected slots are the exact proxy maxima (+inf local, -inf padding)
    seq_of = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1
    for i in range(0, case.total_q, 37):
        s = seq_of[i]
        for g in range(case.cfg.hkv):
            for k, b in enumerate(got[i, g]):
                want = out.scores[s][i - case.cu_q[s], g, b] if b >= 0 else -np.inf
                assert got_sc[i, g, k] == want


@pytest.mark.parametrize("cfgname", ["tiny"])
def test_index_topk_gaussian_certified(cfgname):
    _say(f"[index gaussian] {cfgname}")
    case = mi.make_case(cfgname, seed=0)
    got, _ = gpu_index(case, upload(case))
    out, scores = _oracle_index_scores(case)
    n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, _err_fn(case))
    _say(f"rows differing {n_diff}, certified near-ties {n_tie}")
    assert not bad, f"uncertified list differences at {bad[:5]}"


FP8_INDEX_CASES = [
    # prefill tiles: dp = 64 with block reuse, ragged, causal
    ("tile_dp64", dict(n_q=(1024, 300), n_k=(1024, 2000), hq=8, hkv=2, topk=8, dp=64,
                       lowrank=True)),
    # dp = 32 (zero-filled upper half of the 64-long contraction), non-causal
    ("tile_dp32_noncausal", dict(n_q=(700,), n_k=(3000,), hq=4, hkv=2, topk=6, dp=32,
                                 causal=False)),
    # short-query (key-split) path
    ("split_dp64", dict(n_q=(1, 3), n_k=(5000, 20000), hq=8, hkv=2, topk=16, dp=64)),
    ("split_dp32_noncausal", dict(n_q=(4, 16), n_k=(3000, 7000), hq=8, hkv=4, topk=10, dp=32,
                                  causal=False)),
]


@pytest.mark.parametrize("name,kw", FP8_INDEX_CASES, ids=[c[0] for c in FP8_INDEX_CASES])
def test_index_topk_fp8_bit_exact_on_exact_arithmetic(name, kw):
    """e4m3 proxies holding grid values (codes {-16..16}/4, descale 1): every product is a
    multiple of 2^-4 below 2^4, so the 8-bit MFMA's sums are exact and the lists and scores
    must equal the oracle's bit for bit, ties included."""
    _say(f"[index fp8 exact] {name}")
    kw = dict(kw, proxy="grid")
    kw.pop("lowrank", None)
    case = mi.make_case(mi.custom(name=name, idx_dtype="fp8", **kw), seed=3)
    assert case.idx_descale == (1.0, 1.0)
    got, got_sc = gpu_index(case, upload(case))
    out = msa_case.run(case, want_output=False)
    n_diff, _, bad = compare_lists(got, out.topk_idx)
    assert n_diff == 0, f"{n_diff} rows differ, first {bad[:5]}"
    seq_of = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1
    for i in range(0, case.total_q, 5):
        s = seq_of[i]
        for g in range(case.cfg.hkv):
            for k, b in enumerate(got[i, g]):
                want = out.scores[s][i - case.cu_q[s], g, b] if b >= 0 else -np.inf
                assert got_sc[i, g, k] == want


@pytest.mark.parametrize("name,kw", FP8_INDEX_CASES, ids=[c[0] for c in FP8_INDEX_CASES])
def test_index_topk_fp8_proxies_certified(name, kw):
    """e4m3 proxies: lists equal the oracle's on the dequantised proxies up to certified
    near-ties; reported scores are the oracle's block maxima within the fp32 summation bound."""
    _say(f"[index fp8 proxies] {name}")
    case = mi.make_case(mi.custom(name=name, idx_dtype="fp8", **kw), seed=2)
    got, got_sc = gpu_index(case, upload(case))
    out, scores = _oracle_index_scores(case)
    err = _err_fn(case)
    n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, err)
    _say(f"rows differing {n_diff}, certified near-ties {n_tie}")
    assert not bad, f"uncertified list differences at {bad[:5]}"
    n_checked = 0
    for i in range(0, case.total_q, 7):
        for g in range(case.cfg.hkv):
            for k, b in enumerate(got[i, g]):
                want = scores(i, g)[b] if b >= 0 else -np.inf
                if not np.isfinite(want):
                    assert got_sc[i, g, k] == want
                    continue
                tol = err(i, g)[b] + 2.0 ** -22 * abs(want)    # block b's score bound
                assert abs(got_sc[i, g, k] - want) <= tol, (i, g, k, got_sc[i, g, k], want)
                n_checked += 1
    assert n_checked > 0


MXFP4_INDEX_CASES = FP8_INDEX_CASES + [
    # ragged sequences in one call, one group, a last block of 1 key
    ("tile_ragged_g1", dict(n_q=(300, 129, 700), n_k=(300, 2049, 700), hq=4, hkv=1, topk=9,
                            dp=64)),
    ("split_g8_decode", dict(n_q=(1, 1), n_k=(3000, 12000), hq=16, hkv=8, topk=16, dp=64)),
]


@pytest.mark.parametrize("name,kw", MXFP4_INDEX_CASES, ids=[c[0] for c in MXFP4_INDEX_CASES])
def test_index_topk_mxfp4_bit_exact(name, kw):
    """MXFP4 proxies ("Sparse Attention", Chapter 4: the FP4 scorer): every product of two
    E2M1 values is a multiple of 1/4 below 36, a 32-element group sums exactly, the scales are
    powers of two, so each score is exact whenever its exact value is an fp32 number (checked
    here on the oracle's scores). Lists and scores must then equal the oracle's bit for bit,
    ties included, with no near-tie allowance."""
    _say(f"[index mxfp4] {name}")
    case = mi.make_case(mi.custom(name=name, idx_dtype="mxfp4", **kw), seed=4)
    got, got_sc = gpu_index(case, upload(case))
    out = msa_case.run(case, want_output=False)
    for sc in out.scores:
        fin = sc[np.isfinite(sc)]
        assert np.array_equal(fin.astype(np.float32).astype(np.float64), fin)
    n_diff, _, bad = compare_lists(got, out.topk_idx)
    assert n_diff == 0, f"{n_diff} rows differ, first {bad[:5]}"
    seq_of = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1
    n_checked = 0
    for i in range(0, case.total_q, 3):
        s = seq_of[i]
        for g in range(case.cfg.hkv):
            for k, b in enumerate(got[i, g]):
                want = out.scores[s][i - case.cu_q[s], g, b] if b >= 0 else -np.inf
                assert got_sc[i, g, k] == want, (i, g, k, got_sc[i, g, k], want)
                n_checked += 1
    assert n_checked > 0


# ------------------------------------------------------------------ whole layer

LAYER_CASES = [
    ("tiny", mi.CONFIGS["tiny"], 0),
    ("tiny_seed2", mi.CONFIGS["tiny"], 2),
    ("ragged_varlen", mi.custom(name="ragged", n_q=(300, 1, 640, 129), n_k=(700, 4000, 640, 129),
                                hq=8, hkv=2, topk=5, dp=64), 3),
    ("group4_lowrank", mi.custom(name="g4", n_q=(1024,), hq=16, hkv=4, topk=6, dp=64,
                                 lowrank=True), 0),
    ("noncausal_g1", mi.custom(name="nc", n_q=(256, 200), n_k=(1000, 333), hq=4, hkv=4, topk=4,
                               dp=32, causal=False), 0),
    ("fp8_small", mi.custom(name="fp8", n_q=(1024,), hq=32, hkv=2, topk=6, dp=64, dtype="fp8",
                            lowrank=True), 0),
    ("multi_range", mi.custom(name="mr", n_q=(4500, 700), n_k=(4500, 5000), hq=4, hkv=2, topk=5,
                              dp=32, lowrank=True), 0),
    # group sizes whose Q rows of one 1 KiB load span several queries (bf16: G < 4, fp8: G < 8)
    ("group2", mi.custom(name="g2", n_q=(700, 130), n_k=(700, 1000), hq=4, hkv=2, topk=5,
                         dp=32), 1),
    ("group8", mi.custom(name="g8", n_q=(900,), hq=16, hkv=2, topk=6, dp=64, lowrank=True), 2),
    ("fp8_group4", mi.custom(name="f4", n_q=(800,), hq=8, hkv=2, topk=5, dp=32, dtype="fp8"), 3),
    ("fp8_group1_ragged", mi.custom(name="f1", n_q=(600, 300), n_k=(600, 900), hq=2, hkv=2,
                                    topk=4, dp=32, dtype="fp8"), 4),
    # G = 16 (one entry per tile row group of 16) over ragged causal sequences
    ("group16_ragged", mi.custom(name="g16r", n_q=(700, 257), n_k=(1500, 257), hq=32, hkv=2,
                                 topk=6, dp=64), 1),
    # non-causal, three 512-query ranges with a ragged last one, G = 8
    ("noncausal_g8_ranges", mi.custom(name="nc8", n_q=(1300,), n_k=(2000,), hq=16, hkv=2,
                                      topk=6, dp=32, causal=False), 2),
    # 32 fp8 sequences: the schedule keeps 128 (sequence, group, range) phases by taking
    # 1024-query ranges, two of them in the long sequence, one (or an empty second) elsewhere
    ("fp8_ranges_1024", mi.custom(name="f8mr", n_q=(2048,) + tuple(17 + 11 * i for i in range(31)),
                                  n_k=(2048,) + tuple(17 + 11 * i + (300 if i % 3 == 0 else 0)
                                                      for i in range(31)),
                                  hq=8, hkv=2, topk=5, dp=32, dtype="fp8", lowrank=True), 5),
]


@pytest.mark.parametrize("name,cfg,seed", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
@pytest.mark.parametrize("mode", [msa.MSA_KV_OUTER, msa.MSA_Q_OUTER], ids=["kv", "q"])
def test_layer_matches_oracle(name, cfg, seed, mode):
    _say(f"[layer] {name} mode={mode}")
    case = mi.make_case(cfg, seed=seed)
    dev = upload(case)
    out = msa_case.run(case)
    # main branch on the oracle's own lists (oracle -> GPU direction only)
    lists = torch.from_numpy(out.topk_idx).cuda()
    o, lse = gpu_attention(case, dev, lists, mode)
    tol_o, tol_l = TOL[case.cfg.dtype]
    st = err_stats(o, out.o, lse, out.lse)
    _say(st)
    assert st["max_abs"] <= tol_o and st["max_dlse"] <= tol_l and st["lse_inf_match"]


def test_index_then_layer_end_to_end():
    """The index branch's own lists feed the main branch. Lists: bit-exact, or a certified
    near-tie (capped in number); outputs against the oracle's on every row whose list equals
    the oracle's (a row with a certified swap ran on other lists)."""
    _say("[e2e] tiny")
    case = mi.make_case("tiny", seed=0)
    dev = upload(case)
    got, _ = gpu_index(case, dev)
    out, scores = _oracle_index_scores(case)
    n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, _err_fn(case))
    _say(f"rows differing {n_diff}, certified near-ties {n_tie}")
    assert not bad, f"uncertified list differences at {bad[:5]}"
    ref = msa_case.run(case)
    same = np.all(got == ref.topk_idx, axis=(1, 2))
    o, lse = gpu_attention(case, dev, torch.from_numpy(got).cuda(), msa.MSA_AUTO)
    st = err_stats(o[same], ref.o[same], lse[same], ref.lse[same])
    _say(st, "rows compared", int(same.sum()))
    assert st["max_abs"] <= 2e-2 and st["max_dlse"] <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_partials_match_oracle_partials(dtype):
    """KV-outer partial outputs and LSEs, read through the documented workspace layout."""
    _say(f"[partials] {dtype}")
    case = mi.make_case(mi.custom(name="p", n_q=(512, 300), n_k=(512, 700), hq=8, hkv=2, topk=4,
                                  dp=32, dtype=dtype), seed=5)
    tol_o, tol_l = TOL[dtype]
    dev = upload(case)
    out = msa_case.run(case, want_output=False)
    lists = torch.from_numpy(out.topk_idx).cuda()
    o, lse, ws, s, chosen = gpu_attention(case, dev, lists, msa.MSA_KV_OUTER, keep_ws=True)
    L = msa.msa_workspace_layout_of(s, chosen)
    wsn = ws.cpu()
    G = case.cfg.hq // case.cfg.hkv
    n_ent = int(wsn[L.counters:L.counters + 4].view(torch.int32)[0])
    cmap = wsn[L.cmap:L.cmap + case.total_q * case.cfg.hkv * case.cfg.topk * 4].view(torch.int32)
    cmap = cmap.numpy().reshape(case.total_q, case.cfg.hkv, case.cfg.topk)
    plse = wsn[L.part_lse:L.part_lse + n_ent * G * 4].view(torch.float32).numpy().reshape(n_ent, G)
    pl = wsn[L.part_l:L.part_l + n_ent * G * 4].view(torch.float32).numpy().reshape(n_ent, G)
    # 8-row groups: chunk c (dims 8c..8c+7) of row p at byte ((p // 8) * 16 + c) * 128 + (p % 8) * 16
    n_grp = -(-n_ent * G // 8)
    po = wsn[L.part_o:L.part_o + n_grp * 2048].view(torch.bfloat16).float().numpy()
    po = po.reshape(n_grp, 16, 8, 8).transpose(0, 2, 1, 3).reshape(n_grp * 8, 128)[:n_ent * G]
    # stored unnormalised: output times the weight sum (a block always has a visible key here)
    assert np.all(pl >= 1.0)
    po = po.reshape(n_ent, G, 128) / pl[:, :, None]
    entry_q = wsn[L.entry_q:L.entry_q + n_ent * 4].view(torch.int32).numpy()
    # every valid slot maps to a distinct entry that records its query
    valid = cmap >= 0
    assert np.all((out.topk_idx >= 0) == valid)
    ents = cmap[valid]
    assert len(np.unique(ents)) == ents.size == n_ent
    rows = np.nonzero(valid)[0]
    assert np.array_equal(entry_q[ents], rows)
    dq, dk, dv = case.descale
    q, k, v = widen(case.q, dq), widen(case.k, dk), widen(case.v, dv)
    for si in range(2):
        q0, q1 = case.cu_q[si], case.cu_q[si + 1]
        k0, k1 = case.cu_k[si], case.cu_k[si + 1]
        o_s, l_s = ref.partial_attention(q[q0:q1], k[k0:k1], v[k0:k1], out.topk_idx[q0:q1],
                                         case.softmax_scale, 128, True)
        for i in range(q1 - q0):
            for g in range(case.cfg.hkv):
                for slot in range(case.cfg.topk):
                    e = cmap[q0 + i, g, slot]
                    if e < 0:
                        continue
                    heads = slice(g * G, (g + 1) * G)
                    assert np.max(np.abs(po[e] - o_s[i, heads, slot])) <= tol_o
                    assert np.max(np.abs(plse[e] - l_s[i, heads, slot])) <= tol_l
    # entries are sorted by (sequence, group, query range, block, query) and carry their bucket
    ebk = wsn[L.entry_bucket:L.entry_bucket + n_ent * 4].view(torch.int32).numpy()
    qr = 64 * L.words_per_bucket
    key = []
    for e in range(n_ent):
        t = entry_q[e]
        i_g, i_slot = np.argwhere(cmap[t] == e)[0]
        si = int(np.searchsorted(case.cu_q, t, side="right") - 1)
        rr = (t - case.cu_q[si]) // qr
        blk = out.topk_idx[t, i_g, i_slot]
        key.append((si, i_g, rr, blk, t))
        assert ebk[e] == ((si * case.cfg.hkv + i_g) * L.n_ranges + rr) * L.nb_max + blk
    assert key == sorted(key)


def test_tile_lists_q_outer_and_kv_outer():
    """Per-Q-tile lists (16 of 64 blocks, non-causal), both schedules, against the oracle."""
    _say("[tile lists]")
    cfg = mi.scaled(mi.CONFIGS["qtile"], 1024)
    cfg = mi.Config(**{**cfg.__dict__, "n_k": (8192,), "hq": 4, "hkv": 4})
    case = mi.make_case(cfg, seed=0)
    dev = upload(case)
    out = msa_case.run(case)
    for mode in (msa.MSA_Q_OUTER, msa.MSA_KV_OUTER):
        o, lse = gpu_attention(case, dev, dev.lists, mode)
        st = err_stats(o, out.o, lse, out.lse)
        _say(mode, st)
        assert st["max_abs"] <= 2e-2 and st["max_dlse"] <= 1e-2


TILE_CASES = [
    # causal, varlen with ragged tails, a one-query sequence, blocks past a sequence's end in
    # the pool, G = 2
    ("causal_varlen_g2", mi.custom(name="tc", n_q=(1000, 300, 1), n_k=(1000, 700, 2000), hq=8,
                                   hkv=4, topk=6, causal=True, list_q=128, list_pool=8), 0),
    # non-causal, bottom-right aligned, one KV head for four query heads, long lists
    ("noncausal_g4", mi.custom(name="tn", n_q=(384,), n_k=(2000,), hq=4, hkv=1, topk=12,
                               causal=False, list_q=128, list_pool=15), 1),
    # fp8 Q/K/V on per-tile lists
    ("fp8", mi.custom(name="tf", n_q=(512,), hq=4, hkv=2, topk=4, dtype="fp8", causal=False,
                      list_q=128, list_pool=4), 2),
]


@pytest.mark.parametrize("name,cfg,seed", TILE_CASES, ids=[c[0] for c in TILE_CASES])
def test_tile_lists_edge_cases(name, cfg, seed):
    """Per-tile lists with -1 padding, repeated blocks and out-of-range ids, both schedules."""
    _say(f"[tile lists] {name}")
    case = mi.make_case(cfg, seed=seed)
    rng = np.random.default_rng(seed)
    lists = case.lists
    n_rows = lists.shape[0] * lists.shape[1]
    flat = lists.reshape(n_rows, -1)
    for i in rng.choice(n_rows, max(1, n_rows // 3), replace=False):
        flat[i, -1] = -1                                   # shorter list
    for i in rng.choice(n_rows, max(1, n_rows // 3), replace=False):
        flat[i, 1] = flat[i, 0]                            # a block listed twice
    flat[0, 0] = 10_000                                    # out of range: skipped
    dev = upload(case)
    out = msa_case.run(case)
    tol_o, tol_l = TOL[case.cfg.dtype]
    for mode in (msa.MSA_Q_OUTER, msa.MSA_KV_OUTER):
        o, lse = gpu_attention(case, dev, dev.lists, mode)
        st = err_stats(o, out.o, lse, out.lse)
        _say(mode, st)
        assert st["max_abs"] <= tol_o and st["max_dlse"] <= tol_l and st["lse_inf_match"]


def _mutate_per_query_lists(case, lists, rng):
    """-1 padding, rows with no block at all, repeated blocks, out-of-range ids and blocks
    past the query's local block (every key masked under causality)."""
    out = lists.copy()
    t_q, hkv, k = out.shape
    rows = [(t, g) for t in range(t_q) for g in range(hkv)]
    pick = lambda frac: [rows[i] for i in rng.choice(len(rows), max(1, int(len(rows) * frac)),
                                                     replace=False)]
    for t, g in pick(0.2):
        out[t, g, -1] = -1
    for t, g in pick(0.2):
        out[t, g, 2] = out[t, g, 0]
    for t, g in pick(0.1):
        out[t, g, 1] = 10_000
    seq = np.searchsorted(case.cu_q, np.arange(t_q), side="right") - 1
    for t, g in pick(0.1):
        s = seq[t]
        n_q = case.cu_q[s + 1] - case.cu_q[s]
        n_k = case.cu_k[s + 1] - case.cu_k[s]
        loc = (n_k - n_q + t - case.cu_q[s]) // 128
        if loc + 1 < -(-n_k // 128):
            out[t, g, 3] = loc + 1
    for t, g in pick(0.05):
        out[t, g, :] = -1
    return out


def test_per_query_lists_edge_cases_and_empty_sequence():
    """A batch with an empty sequence between two ragged ones: the index branch on it, then
    both schedules on per-query lists with degenerate entries, against the oracle on the
    same lists."""
    _say("[per-query list edges]")
    cfg = mi.custom(name="pq", n_q=(400, 0, 333), n_k=(400, 200, 900), hq=8, hkv=2, topk=5,
                    dp=32)
    case = mi.make_case(cfg, seed=7)
    dev = upload(case)
    got, _ = gpu_index(case, dev)
    out, scores = _oracle_index_scores(case)
    n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, _err_fn(case))
    assert not bad, f"uncertified list differences at {bad[:5]}"
    lists = _mutate_per_query_lists(case, out.topk_idx, np.random.default_rng(7))
    ref = msa_case.run(case, lists=lists)
    assert np.any(np.isneginf(ref.lse))                     # rows with no visible key
    for mode in (msa.MSA_KV_OUTER, msa.MSA_Q_OUTER):
        o, lse = gpu_attention(case, dev, torch.from_numpy(lists).cuda(), mode)
        st = err_stats(o, ref.o, lse, ref.lse)
        _say(mode, st)
        assert st["max_abs"] <= 2e-2 and st["max_dlse"] <= 1e-2 and st["lse_inf_match"]


def test_zero_queries_leave_outputs_untouched():
    """total_q = 0: every entry point succeeds and writes nothing."""
    _say("[zero queries]")
    case = mi.make_case(mi.custom(name="z", n_q=(0,), n_k=(256,), hq=4, hkv=2, topk=3, dp=32),
                        seed=1)
    dev = upload(case)
    s = shape_of(case)
    lists = torch.full((1, 2, 3), -7, dtype=torch.int32, device="cuda")
    iws = torch.empty(max(msa.msa_index_workspace_size(s), 256), dtype=torch.uint8, device="cuda")
    msa.msa_index_topk(s, dev.q_idx, dev.k_idx, dev.cu_q, dev.cu_k, lists, None, iws)
    o = torch.full((1, 4, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 4), 3.0, dtype=torch.float32, device="cuda")
    for mode in (msa.MSA_KV_OUTER, msa.MSA_Q_OUTER):
        ws = torch.zeros(max(msa.msa_workspace_size(s, mode), 256), dtype=torch.uint8,
                         device="cuda")
        msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, dev.descale, case.softmax_scale, lists,
                                dev.cu_q, dev.cu_k, mode, ws, o, lse)
        msa.msa_combine(s, mode, ws, o, lse)
    torch.cuda.synchronize()
    assert torch.all(lists == -7) and torch.all(o == 3.0) and torch.all(lse == 3.0)


def test_decode_q_outer_splits():
    _say("[decode]")
    cfg = mi.Config(name="dec", batch=6, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
                    length_seed_draw=(6, 16, 40))
    case = mi.make_case(cfg, seed=0)
    dev = upload(case)
    got, _ = gpu_index(case, dev)
    out, scores = _oracle_index_scores(case)
    n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, _err_fn(case))
    assert not bad
    full = msa_case.run(case)
    for mode in (msa.MSA_AUTO, msa.MSA_KV_OUTER):
        o, lse = gpu_attention(case, dev, torch.from_numpy(full.topk_idx).cuda(), mode)
        st = err_stats(o, full.o, lse, full.lse)
        _say(mode, st)
        assert st["max_abs"] <= 2e-2 and st["max_dlse"] <= 1e-2


def test_bitwise_deterministic():
    _say("[determinism]")
    case = mi.make_case(mi.custom(name="det", n_q=(1024,), hq=16, hkv=2, topk=8, dp=64,
                                  lowrank=True), seed=4)
    dev = upload(case)
    a_idx, _ = gpu_index(case, dev)
    b_idx, _ = gpu_index(case, dev)
    assert np.array_equal(a_idx, b_idx)
    lists = torch.from_numpy(a_idx).cuda()
    for mode in (msa.MSA_KV_OUTER, msa.MSA_Q_OUTER):
        o1, l1 = gpu_attention(case, dev, lists, mode)
        o2, l2 = gpu_attention(case, dev, lists, mode)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_constant_values_and_invariants():
    """V = 1 gives O = 1 within one bf16 ulp; the local block sits in slot 0."""
    _say("[invariants]")
    case = mi.make_case(mi.custom(name="inv", n_q=(640,), hq=8, hkv=2, topk=3, dp=32), seed=6)
    case.v = torch.ones_like(case.v)
    dev = upload(case)
    got, _ = gpu_index(case, dev)
    assert np.all(got[:, :, 0] == (np.arange(640) // 128)[:, None])
    for mode in (msa.MSA_KV_OUTER, msa.MSA_Q_OUTER):
        o, _ = gpu_attention(case, dev, torch.from_numpy(got).cuda(), mode)
        assert np.max(np.abs(o - 1.0)) <= 2 ** -7


@pytest.mark.parametrize("mode", [msa.MSA_KV_OUTER, msa.MSA_Q_OUTER], ids=["kv", "q"])
def test_topk1_local_only_is_block_diagonal_attention(mode):
    """topK = 1: the index branch keeps only the forced local block, so the layer is causal
    attention masked to the query's own 128-key block. The GPU index branch and main branch
    run end to end; the lists must be exactly the local block, and the output is compared
    with torch's scaled_dot_product_attention (CPU, float64) under the block-diagonal causal
    mask, computed independently of the oracle."""
    _say(f"[topk=1] mode={mode}")
    case = mi.make_case(mi.custom(name="k1", n_q=(700,), hq=8, hkv=2, topk=1, dp=32), seed=8)
    dev = upload(case)
    got, _ = gpu_index(case, dev)
    n = case.total_q
    assert np.array_equal(got[:, :, 0], np.repeat((np.arange(n) // 128)[:, None], 2, axis=1))
    o, lse = gpu_attention(case, dev, torch.from_numpy(got).cuda(), mode)
    q = torch.from_numpy(widen(case.q)).permute(1, 0, 2)                      # [Hq, N, D]
    kv_rep = case.cfg.hq // case.cfg.hkv
    k = torch.from_numpy(widen(case.k)).permute(1, 0, 2).repeat_interleave(kv_rep, dim=0)
    v = torch.from_numpy(widen(case.v)).permute(1, 0, 2).repeat_interleave(kv_rep, dim=0)
    i = torch.arange(n)
    mask = (i[None, :] <= i[:, None]) & (i[None, :] // 128 == i[:, None] // 128)
    want = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=case.softmax_scale).permute(1, 0, 2).numpy()
    err = float(np.max(np.abs(o - want)))
    _say(f"max |O - O_sdpa| = {err:.3e}")
    assert err <= 2e-2
