"""Full-size workloads, in the call sequence the benchmark times, against the fp64 oracle.

The oracle cannot score every query of a 32K- or 128K-token layer in test time, so each
workload is checked on a seeded systematic sample of whole 128-query blocks (lists bit-exact
up to certified near-ties, capped in number; outputs at the bf16 / fp8 bars on the sampled
rows whose lists equal the oracle's), and on
properties that hold for every row at any size: the local block fills slot 0, a row holds
min(topK, c + 1) distinct visible blocks followed by -1 padding, and every output is finite.
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case
from synth import msa_inputs as mi

from gpu_util import (compare_lists, err_stats, proxies, proxy_score_errors, run_index,
                      shape_of, upload)

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-2), "fp8": (6e-2, 5e-2)}


def _say(*a):
    print(*a, flush=True)


def bench_sequence(case, dev):
    """index -> plan -> KV-outer attention -> combine (or the Q-outer call), as timed."""
    s = shape_of(case)
    chosen = msa.msa_resolve_mode(s, msa.MSA_AUTO)
    c = case.cfg
    if dev.lists is None:
        lists = torch.full((case.total_q, c.hkv, c.topk), -7, dtype=torch.int32, device="cuda")
        iws = torch.empty(max(msa.msa_index_workspace_size(s), 256), dtype=torch.uint8,
                          device="cuda")
        run_index(case, dev, s, lists, None, iws)
    else:
        lists = dev.lists
    ws = torch.empty(msa.msa_workspace_size(s, chosen), dtype=torch.uint8, device="cuda")
    o = torch.full((case.total_q, c.hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.total_q, c.hq), float("nan"), dtype=torch.float32, device="cuda")
    if chosen == msa.MSA_KV_OUTER:
        msa.msa_plan(s, lists, dev.cu_q, dev.cu_k, ws)
        msa.msa_attn_main(s, dev.q, dev.k, dev.v, dev.descale, case.softmax_scale, dev.cu_q,
                          dev.cu_k, ws)
    else:
        msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, dev.descale, case.softmax_scale, lists,
                                dev.cu_q, dev.cu_k, chosen, ws, o, lse)
    msa.msa_combine(s, chosen, ws, o, lse)
    torch.cuda.synchronize()
    del ws
    return chosen, lists.cpu().numpy(), o, lse


def check_list_properties(case, lists):
    """Every row: local block in slot 0, min(K, c+1) distinct visible blocks, then -1."""
    c = case.cfg
    for s in range(len(case.cu_q) - 1):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        nk = int(case.cu_k[s + 1] - case.cu_k[s])
        pos = nk - (q1 - q0) + np.arange(q1 - q0)
        loc = pos // 128
        lst = lists[q0:q1].astype(np.int64)                      # [n, hkv, K]
        assert np.all(lst[:, :, 0] == loc[:, None])
        count = np.minimum(c.topk, loc + 1)
        valid = lst >= 0
        assert np.all(valid.sum(axis=2) == count[:, None])
        # valid slots come first
        assert np.all(np.diff(valid.astype(np.int8), axis=2) <= 0)
        assert np.all(np.where(valid, lst <= loc[:, None, None], True))
        srt = np.sort(np.where(valid, lst, -1 - np.arange(c.topk)), axis=2)
        assert np.all(np.diff(srt, axis=2) != 0)


def run_workload(cfgname, every, seed=0, max_rows=None):
    _say(f"[full-size] {cfgname}: generating")
    case = mi.make_case(cfgname, seed=seed)
    dev = upload(case)
    _say(f"[full-size] {cfgname}: GPU layer call")
    chosen, lists, o, lse = bench_sequence(case, dev)
    rows = msa_case.sample_rows(case, every=every, seed=seed)
    if max_rows is not None:
        rows = rows[:max_rows]
    o_s = o[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    lse_s = lse[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert torch.isfinite(o.float()).all() and not torch.isnan(lse).any()
    del dev, o, lse
    torch.cuda.empty_cache()
    _say(f"[full-size] {cfgname}: oracle on {rows.size} rows")
    out = msa_case.run(case, rows=rows)
    return case, chosen, lists, rows, out, o_s, lse_s


def compare(case, lists, rows, out, o_s, lse_s, exact_lists=False):
    """Sampled rows: lists bit-exact or certified near-ties (capped in number); outputs
    against the oracle's on every sampled row whose list equals the oracle's."""
    c = case.cfg
    ref_o, ref_lse = out.o, out.lse
    if case.lists is None:
        check_list_properties(case, lists)
        seq_of = np.searchsorted(case.cu_q, rows, side="right") - 1
        qi, ki = proxies(case)

        seqs = np.unique(seq_of)          # the oracle keeps scores of sampled sequences only

        def scores(n, g):
            s = seq_of[n]
            sc = out.scores[int(np.searchsorted(seqs, s))]
            # scores of sequence s are stored for its sampled rows in order
            first = np.searchsorted(seq_of, s)
            return sc[n - first, g]

        def err(n, g):
            s = seq_of[n]
            k0, k1 = case.cu_k[s], case.cu_k[s + 1]
            pos = (k1 - k0) - (case.cu_q[s + 1] - case.cu_q[s]) + (rows[n] - case.cu_q[s])
            return proxy_score_errors(qi[rows[n], g], ki[k0:k1, g],
                                      int(pos) if c.causal else None, c.idx_dtype == "fp8")

        got = lists[rows]
        n_diff, n_tie, bad = compare_lists(got, out.topk_idx, scores, err)
        _say(f"rows differing {n_diff}, certified near-ties {n_tie} of {got.shape[0] * c.hkv}")
        assert not bad, f"uncertified list differences at {bad[:5]}"
        if exact_lists:
            assert n_diff == 0, f"{n_diff} (row, group) lists differ"
        # rows with a certified swap ran on other lists than the oracle's: left out
        same = np.all(got == out.topk_idx, axis=(1, 2))
    else:
        same = np.ones(rows.size, dtype=bool)
    tol_o, tol_l = TOL[c.dtype]
    st = err_stats(o_s[same], ref_o[same], lse_s[same], ref_lse[same])
    _say(st, "rows compared", int(same.sum()), "of", rows.size)
    assert st["max_abs"] <= tol_o and st["max_dlse"] <= tol_l and st["lse_inf_match"]


def test_m3_prefill_32k():
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("m3", every=32)
    assert chosen == msa.MSA_KV_OUTER
    compare(case, lists, rows, out, o_s, lse_s)


def test_fp8_prefill_128k():
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("m3_fp8_long", every=64)
    assert chosen == msa.MSA_KV_OUTER
    compare(case, lists, rows, out, o_s, lse_s)


def test_fp8_proxies_prefill_128k():
    """The 128K fp8 workload with its proxies quantised to e4m3 too (8-bit MFMA scoring)."""
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("m3_fp8_long_i8", every=64)
    assert chosen == msa.MSA_KV_OUTER
    compare(case, lists, rows, out, o_s, lse_s)


def test_mxfp4_proxies_prefill_128k():
    """The 128K fp8 workload with 4-bit MXFP4 proxies: exact scores, so the lists must equal
    the oracle's on every sampled row, with no near-tie allowance."""
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("m3_fp8_long_i4", every=64)
    assert chosen == msa.MSA_KV_OUTER
    compare(case, lists, rows, out, o_s, lse_s, exact_lists=True)


def test_mxfp4_proxies_decode_64_requests():
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("decode_i4", every=1)
    assert chosen == msa.MSA_Q_OUTER
    compare(case, lists, rows, out, o_s, lse_s, exact_lists=True)


def test_decode_64_requests():
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("decode", every=1)
    assert chosen == msa.MSA_Q_OUTER
    compare(case, lists, rows, out, o_s, lse_s)


def test_per_q_tile_lists_8k():
    case, chosen, lists, rows, out, o_s, lse_s = run_workload("qtile", every=16)
    assert chosen == msa.MSA_Q_OUTER
    compare(case, lists, rows, out, o_s, lse_s)
