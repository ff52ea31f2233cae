"""Per-Q-tile block selectors R1 / R4 ("Sparse Attention", Chapter 4) on the GPU against the
fp64 oracle, and the selector -> per-tile attention pipeline.

Lists must equal the oracle's up to certified near-ties: the GPU averages bf16 tokens and
forms the dot products in fp32, so a representative's error is within gamma_128 of the mean
of |x| per dimension and a score's within 3 gamma_128 sum_d A_d B_d (A, B: means of |q|,
|k|); each block's score is taken within 4 gamma_128 |A|_2 |B|_2 of the oracle's, and a
differing list must be the selection of some scores within those bounds (capped in number)."""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case, selectors as S
from synth import msa_inputs as mi
from synth.msa_inputs import widen

from gpu_util import compare_lists, err_stats, gpu_attention, shape_of, upload

pytestmark = pytest.mark.gpu
GAMMA = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)


def _say(*a):
    print(*a, flush=True)


def oracle_select(case, reps):
    """Per-tile lists [B * tiles_max, Hkv, K] and, per (row, group), the oracle's block
    scores and the near-tie bound."""
    c = case.cfg
    g_size = c.hq // c.hkv
    q, k = widen(case.q), widen(case.k)
    tiles_max = -(-case.max_q // 128)
    n_seq = len(case.cu_q) - 1
    lists = np.full((n_seq * tiles_max, c.hkv, c.topk), -1, dtype=np.int32)
    scores, bounds = {}, {}
    for s in range(n_seq):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        k0, k1 = int(case.cu_k[s]), int(case.cu_k[s + 1])
        if q1 == q0:
            continue
        lst, sc = S.select_tiles(q[q0:q1], k[k0:k1], reps, 128, g_size, c.topk, c.causal)
        lists[s * tiles_max:s * tiles_max + lst.shape[0]] = lst
        a = S.representatives(np.abs(q[q0:q1]), reps, 128)
        b = S.representatives(np.abs(k[k0:k1]), reps, 128)
        for t in range(lst.shape[0]):
            for g in range(c.hkv):
                na = np.nanmax(np.linalg.norm(a[t, g * g_size:(g + 1) * g_size], axis=-1))
                nb = np.nanmax(np.linalg.norm(b[:, g], axis=-1)) if b.shape[0] else 0.0
                scores[(s * tiles_max + t, g)] = sc[t, g]
                bounds[(s * tiles_max + t, g)] = 2 * 4 * GAMMA * na * nb
    return lists, scores, bounds


def gpu_select(case, dev, reps):
    s = shape_of(case)
    tiles_max = -(-case.max_q // 128)
    rows = (len(case.cu_q) - 1) * tiles_max
    lists = torch.full((rows, case.cfg.hkv, case.cfg.topk), -7, dtype=torch.int32,
                       device="cuda")
    sc = torch.full(lists.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(msa.msa_select_workspace_size(s, reps), dtype=torch.uint8, device="cuda")
    msa.msa_select_tiles(s, reps, dev.q, dev.k, dev.cu_q, dev.cu_k, lists, sc, ws)
    torch.cuda.synchronize()
    return lists, sc.cpu().numpy()


SEL_CASES = [
    # G = 16 (a block's 256 pairs span four waves), ragged tiles and blocks, two sequences
    ("g16_r4", dict(n_q=(700, 300), n_k=(3000, 1000), hq=16, hkv=1, topk=8, causal=False), 4),
    ("g16_r1", dict(n_q=(700, 300), n_k=(3000, 1000), hq=16, hkv=1, topk=8, causal=False), 1),
    # causal visibility, G = 4 (64 pairs: one wave per block)
    ("g4_causal_r4", dict(n_q=(1000,), n_k=(1500,), hq=8, hkv=2, topk=6, causal=True), 4),
    # G = 8 (128 pairs: two waves per block), more blocks than chunk and list
    ("g8_r4", dict(n_q=(384,), n_k=(5000,), hq=16, hkv=2, topk=16, causal=False), 4),
    # G = 2 (32 pairs) and G = 1 with R1 (one pair: 256 blocks per pass), fewer blocks than K
    ("g2_r4", dict(n_q=(300,), n_k=(2000,), hq=4, hkv=2, topk=5, causal=False), 4),
    ("g1_r1_short", dict(n_q=(256, 129), n_k=(600, 1000), hq=2, hkv=2, topk=12, causal=True), 1),
]


@pytest.mark.parametrize("name,kw,reps", SEL_CASES, ids=[c[0] for c in SEL_CASES])
def test_selector_matches_oracle(name, kw, reps):
    _say(f"[selector] {name}")
    case = mi.make_case(mi.custom(name=name, list_q=128, selector=reps, **kw), seed=4)
    dev = upload(case)
    got, got_sc = gpu_select(case, dev, reps)
    got = got.cpu().numpy()
    want, scores, bounds = oracle_select(case, reps)
    n_diff, n_tie, bad = compare_lists(got, want, lambda i, g: scores[(i, g)],
                                       lambda i, g: bounds[(i, g)] / 2)
    _say(f"rows differing {n_diff}, certified near-ties {n_tie}")
    assert not bad, f"uncertified list differences at {bad[:5]}"
    # reported scores: the oracle's within one score's bound; -inf on empty slots
    for (i, g), sc in scores.items():
        for slot, b in enumerate(got[i, g]):
            if b < 0:
                assert got_sc[i, g, slot] == -np.inf
            else:
                assert abs(got_sc[i, g, slot] - sc[b]) <= bounds[(i, g)] / 2 + 1e-6 * abs(sc[b])
    # rows past a sequence's tiles hold -1
    assert np.all(got[[r for r in range(got.shape[0]) if all((r, g) not in scores
                                                              for g in range(case.cfg.hkv))]]
                  == -1)


@pytest.mark.parametrize("reps", [1, 4])
def test_selector_then_tile_attention(reps):
    """R1 / R4 lists feed the per-tile attention; lists against the oracle's (exact or
    certified near-ties, capped), outputs against the oracle's on the queries whose tile
    lists equal the oracle's."""
    _say(f"[selector pipeline] R{reps}")
    case = mi.make_case(mi.custom(name="sp", n_q=(640, 200), n_k=(2500, 900), hq=8, hkv=2,
                                  topk=6, causal=False, list_q=128, selector=reps), seed=6)
    dev = upload(case)
    got, _ = gpu_select(case, dev, reps)
    want, scores, bounds = oracle_select(case, reps)
    g_np = got.cpu().numpy()
    n_diff, n_tie, bad = compare_lists(g_np, want, lambda i, g: scores[(i, g)],
                                       lambda i, g: bounds[(i, g)] / 2)
    assert not bad
    _say(f"rows differing {n_diff}, certified near-ties {n_tie}")
    case.lists = want
    out = msa_case.run(case)
    o, lse = gpu_attention(case, dev, got, msa.MSA_AUTO)
    # queries of tiles with a certified swap ran on other lists than the oracle's: left out
    tiles_max = -(-case.max_q // 128)
    same_row = np.all(g_np == want, axis=(1, 2))
    seq = np.searchsorted(case.cu_q, np.arange(case.total_q), side="right") - 1
    keep = same_row[seq * tiles_max + (np.arange(case.total_q) - case.cu_q[seq]) // 128]
    st = err_stats(o[keep], out.o[keep], lse[keep], out.lse[keep])
    _say(st, "queries compared", int(keep.sum()))
    assert st["max_abs"] <= 2e-2 and st["max_dlse"] <= 1e-2 and st["lse_inf_match"]
