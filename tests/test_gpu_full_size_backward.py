"""Main-branch and proxy backward at the full M3 shape (32K causal, Hq = 64, Hkv = 4, top-16),
in the call sequence a training step runs: index -> forward -> backward.

The oracle's index branch is run on every row (one matmul per 512-row chunk and group), which
gives three checks:

* the GPU index branch's lists against the oracle's on all 131,072 (row, group) pairs
  (bit-exact, or a certified near-tie, capped in number);
* the forward and both backward passes on the GPU take the oracle's lists (oracle -> GPU
  direction only), so every compared gradient has the same lists on both sides;
* dK, dV and dk_idx element by element on sampled (group, block) columns, each built by the
  oracle from the queries whose lists hold the block (a column at the 90th percentile of
  queries per column, a causal diagonal column and seeded others); dQ, dq_idx and the proxy LSE on a seeded sample of
  whole 128-query blocks.

Bars, as in the small-case backward tests: per tensor, max |G - G_ref| <= 2e-2 max |G_ref|
and rms(G - G_ref) <= 1e-2 rms(G_ref); proxy LSE within 1e-3. Column sums over every key
are kept as a property at any size: summed over all keys of a group, dV equals the sum of dO
over the group's rows (each row's weights sum to one, within 2^-8 per weight, unbiased: eight
standard deviations, 8 * 2^-8 * sqrt(sum dO^2) per (group, dim)) and dK vanishes (each row's
dS sums to zero; 2e-3 of sum |dK|).

The proxy objective is a reading of the pages (parity unpinned against the pages): these
checks pin the GPU to the oracle of that reading.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case
from oracle.msa_backward import key_block_gradient, query_rows_gradient
from oracle.msa_proxy_backward import proxy_key_block_gradient, proxy_rows_gradient
from synth import msa_inputs as mi
from synth.msa_inputs import widen

from gpu_util import compare_lists, gpu_index, proxies, proxy_score_errors, shape_of, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _check(name, got, want):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - want)
    mx, rms = float(d.max()), float(np.sqrt(np.mean(d ** 2)))
    ref_max, ref_rms = float(np.abs(want).max()), float(np.sqrt(np.mean(want ** 2)))
    _say(f"  {name}: max |d| {mx:.3e} (ref max {ref_max:.3e}), rms {rms:.3e} "
         f"(ref rms {ref_rms:.3e})")
    assert mx <= 2e-2 * ref_max and rms <= 1e-2 * ref_rms, name


def test_m3_backward_32k():
    _say("[full-size backward] m3: generating")
    case = mi.make_case("m3", seed=0)
    c = case.cfg
    n = case.total_q
    _say("[full-size backward] m3: oracle index branch on every row")
    ref = msa_case.run(case, want_output=False)
    lists = ref.topk_idx                                     # [N, Hkv, K], rows 0..N-1
    assert ref.rows.size == n and np.array_equal(ref.rows, np.arange(n))

    dev = upload(case)
    _say("[full-size backward] m3: GPU index branch, all rows against the oracle")
    got, _ = gpu_index(case, dev)
    qi, ki = proxies(case)
    scores = ref.scores[0]

    def err(i, g):
        return proxy_score_errors(qi[i, g], ki[:, g], int(i), False)

    n_diff, n_tie, bad = compare_lists(got, lists, lambda i, g: scores[i, g], err)
    _say(f"  lists: rows differing {n_diff}, certified near-ties {n_tie} of {n * c.hkv}")
    assert not bad, f"uncertified list differences at {bad[:5]}"

    _say("[full-size backward] m3: GPU forward and backward on the oracle's lists")
    s = shape_of(case)
    lists_dev = torch.from_numpy(lists).cuda()
    ws = torch.empty(msa.msa_workspace_size(s, msa.MSA_KV_OUTER), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((n, c.hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((n, c.hq), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, None, case.softmax_scale, lists_dev,
                            dev.cu_q, dev.cu_k, msa.MSA_KV_OUTER, ws, o, lse)
    msa.msa_combine(s, msa.MSA_KV_OUTER, ws, o, lse)
    del ws
    dout = mi.grad_output(case)
    pscale = 1.0 / math.sqrt(c.dp)
    tws = torch.empty(msa.msa_train_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    dq = torch.empty((n, c.hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((case.total_k, c.hkv, 128), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    dqi = torch.empty((n, c.hkv, c.dp), dtype=torch.float32, device="cuda")
    dki = torch.empty((case.total_k, c.hkv, c.dp), dtype=torch.float32, device="cuda")
    lsep = torch.empty((n, c.hkv), dtype=torch.float32, device="cuda")
    msa.msa_train_bwd(s, dev.q, dev.k, dev.v, o, lse, dout.cuda(), case.softmax_scale,
                      dev.q_idx, dev.k_idx, pscale, lists_dev, dev.cu_q, dev.cu_k, tws,
                      dq, dk, dv, dqi, dki, lsep)
    # the proxy-only call gives the same proxy gradients bit for bit
    pws = torch.empty(msa.msa_proxy_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    dqi_p = torch.empty_like(dqi)
    dki_p = torch.empty_like(dki)
    msa.msa_proxy_attn_bwd(s, dev.q, dev.k, dev.q_idx, dev.k_idx, lse, case.softmax_scale,
                           pscale, lists_dev, dev.cu_q, dev.cu_k, pws, dqi_p, dki_p)
    torch.cuda.synchronize()
    assert torch.equal(dqi, dqi_p) and torch.equal(dki, dki_p)
    del tws, pws, o, lse, dev, dqi_p, dki_p
    to_np = lambda t: t.cpu().numpy().astype(np.float64)
    dq_n, dk_n, dv_n, dqi_n, dki_n, lsep_n = map(to_np, (dq, dk, dv, dqi, dki, lsep))
    del dq, dk, dv, dqi, dki, lsep
    torch.cuda.empty_cache()
    for name, t in (("dQ", dq_n), ("dK", dk_n), ("dV", dv_n), ("dq_idx", dqi_n),
                    ("dk_idx", dki_n)):
        assert np.all(np.isfinite(t)), name

    # column sums over every key (one sequence; every row sees its local block)
    do64 = widen(dout)
    for g in range(c.hkv):
        heads = slice(g * (c.hq // c.hkv), (g + 1) * (c.hq // c.hkv))
        want_v = do64[:, heads].sum(axis=(0, 1))
        bound_v = 8 * 2.0 ** -8 * np.sqrt((do64[:, heads] ** 2).sum(axis=(0, 1)))
        err_v = np.abs(dv_n[:, g].sum(axis=0) - want_v)
        err_k = np.abs(dk_n[:, g].sum(axis=0))
        bound_k = 2e-3 * np.abs(dk_n[:, g]).sum(axis=0)
        _say(f"  group {g}: max |sum dV - sum dO| {err_v.max():.3e} (bound {bound_v.min():.3e}), "
             f"max |sum dK| {err_k.max():.3e} (bound {bound_k.min():.3e})")
        assert np.all(err_v <= bound_v) and np.all(err_k <= bound_k)

    q, k, v = widen(case.q), widen(case.k), widen(case.v)
    qi64, ki64 = widen(case.q_idx), widen(case.k_idx)

    # sampled rows: dQ, dq_idx, proxy LSE
    rows = msa_case.sample_rows(case, every=64, seed=0)
    _say(f"[full-size backward] m3: oracle rows ({rows.size})")
    want_dq = query_rows_gradient(q, k, v, lists[rows], do64[rows], rows, case.softmax_scale,
                                  c.block, c.causal)
    _check("dQ rows", dq_n[rows], want_dq)
    want_dqi, want_lp = proxy_rows_gradient(q, k, qi64, ki64, lists[rows], rows,
                                            case.softmax_scale, pscale, c.block, c.causal)
    _check("dq_idx rows", dqi_n[rows], want_dqi)
    assert np.abs(lsep_n[rows] - want_lp).max() <= 1e-3

    # sampled columns: one at the 90th percentile of queries per column (split into several
    # 4096-row chunks whose partial sums are added in order), a causal diagonal one (the
    # last block, whose queries see part of it), and seeded others
    nb = -(-case.total_k // c.block)
    counts = np.zeros((c.hkv, nb), dtype=np.int64)
    for g in range(c.hkv):
        valid = lists[:, g][lists[:, g] >= 0]
        counts[g] = np.bincount(valid, minlength=nb)
    p90 = np.percentile(counts, 90)
    g0, b0 = np.unravel_index(int(np.argmin(np.abs(counts - p90))), counts.shape)
    rng = np.random.default_rng(11)
    cols = [(int(g0), int(b0)), (1, nb - 1)]
    while len(cols) < 6:
        gb = (int(rng.integers(0, c.hkv)), int(rng.integers(0, nb)))
        if gb not in cols:
            cols.append(gb)
    got_k, got_v, got_ki, want_k, want_v, want_ki = [], [], [], [], [], []
    for g, b in cols:
        _say(f"[full-size backward] m3: oracle column (group {g}, block {b}): "
             f"{counts[g, b]} queries")
        wk, wv = key_block_gradient(q, k, v, lists, do64, g, b, case.softmax_scale, c.block,
                                    c.causal)
        wki = proxy_key_block_gradient(q, k, qi64, ki64, lists, g, b, case.softmax_scale,
                                       pscale, c.block, c.causal)
        lo = b * c.block
        hi = lo + wk.shape[0]
        got_k.append(dk_n[lo:hi, g])
        got_v.append(dv_n[lo:hi, g])
        got_ki.append(dki_n[lo:hi, g])
        want_k.append(wk)
        want_v.append(wv)
        want_ki.append(wki)
    _check("dK columns", np.concatenate(got_k), np.concatenate(want_k))
    _check("dV columns", np.concatenate(got_v), np.concatenate(want_v))
    _check("dk_idx columns", np.concatenate(got_ki), np.concatenate(want_ki))
