"""Proxy backward on the GPU (libmsa through its C ABI) against the fp64 oracle.

Both sides take the oracle index branch's lists (or the case's per-tile lists) and the same
bf16 Q, K and proxies; the GPU consumes the GPU forward's LSE. Bar, from the arithmetic: the
main weights P and the proxy weights Pp are fp32 exponentials of fp32 MFMA sums, dz is rounded
to bf16 (relative 2^-9) before the two products, which accumulate in fp32; per tensor
max |G - G_ref| <= 2e-2 max |G_ref| and rms(G - G_ref) <= 1e-2 rms(G_ref); the proxy LSE
within 1e-3.

Parity unpinned against the pages: the objective (KL of the proxy softmax to the
head-averaged main weights over the selected keys) is a reading; the pages print neither it
nor any gradient value. These tests pin the GPU to the oracle of that reading only.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case, msa_proxy_backward
from synth import msa_inputs as mi

from gpu_util import shape_of, upload

pytestmark = pytest.mark.gpu

CASES = [
    ("g16_dp64_causal", dict(n_q=(700,), n_k=(700,), hq=16, hkv=1, topk=4, dp=64)),
    ("g4_dp32_ragged", dict(n_q=(300, 1, 129), n_k=(700, 4000, 129), hq=8, hkv=2, topk=5,
                            dp=32)),
    ("g1_dp64_noncausal", dict(n_q=(200, 384), n_k=(1000, 384), hq=2, hkv=2, topk=6, dp=64,
                               causal=False)),
    ("g8_dp64_split_columns", dict(n_q=(1100,), n_k=(512,), hq=8, hkv=1, topk=4, dp=64,
                                   causal=False)),
    ("g2_dp32_tile_lists", dict(n_q=(384, 200), n_k=(1024, 640), hq=4, hkv=2, topk=4, dp=32,
                                list_q=128, list_pool=8)),
]


def _say(*a):
    print(*a, flush=True)


def _check(name, got, want):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - want)
    mx, rms = float(d.max()), float(np.sqrt(np.mean(d ** 2)))
    ref_max, ref_rms = float(np.abs(want).max()), float(np.sqrt(np.mean(want ** 2)))
    _say(f"  {name}: max |d| {mx:.3e} (ref max {ref_max:.3e}), rms {rms:.3e} (ref rms {ref_rms:.3e})")
    assert mx <= 2e-2 * ref_max + 1e-7 and rms <= 1e-2 * ref_rms + 1e-8, name


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_proxy_backward_matches_oracle(name, kw):
    cfg = mi.custom(name, **kw)
    case = mi.make_case(cfg, seed=13, with_proxies=True)
    pscale = 1.0 / math.sqrt(cfg.dp)
    _say(f"[proxy backward] {name}: total_q {case.total_q} hq {cfg.hq} hkv {cfg.hkv} dp {cfg.dp}")
    sel = msa_case.run(case, want_output=False)
    lists = np.full((case.total_q, cfg.hkv, cfg.topk), -1, dtype=np.int32)
    lists[sel.rows] = sel.topk_idx
    dqi_r, dki_r, _, lsep_r = msa_proxy_backward.run_case(case, lists, pscale)
    dev = upload(case)
    s = shape_of(case)
    lists_dev = torch.from_numpy(lists).cuda() if cfg.list_q == 1 else dev.lists
    ws_f = torch.zeros(msa.msa_workspace_size(s, msa.MSA_KV_OUTER), dtype=torch.uint8,
                       device="cuda")
    o = torch.empty((case.total_q, cfg.hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.total_q, cfg.hq), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, None, case.softmax_scale, lists_dev, dev.cu_q,
                            dev.cu_k, msa.MSA_KV_OUTER, ws_f, o, lse)
    msa.msa_combine(s, msa.MSA_KV_OUTER, ws_f, o, lse)
    ws = torch.empty(msa.msa_proxy_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    dqi = torch.full((case.total_q, cfg.hkv, cfg.dp), float("nan"), device="cuda")
    dki = torch.full((case.total_k, cfg.hkv, cfg.dp), float("nan"), device="cuda")
    lsep = torch.full((case.total_q, cfg.hkv), float("nan"), device="cuda")
    msa.msa_proxy_attn_bwd(s, dev.q, dev.k, dev.q_idx, dev.k_idx, lse, case.softmax_scale,
                           pscale, lists_dev, dev.cu_q, dev.cu_k, ws, dqi, dki, lsep)
    torch.cuda.synchronize()
    lp = lsep.cpu().numpy()
    fin = np.isfinite(lsep_r)
    assert np.all(np.isneginf(lp[~fin])) and np.abs(lp[fin] - lsep_r[fin]).max() <= 1e-3
    _check("dq_idx", dqi.cpu().numpy(), dqi_r)
    _check("dk_idx", dki.cpu().numpy(), dki_r)

    # both passes in one call: main gradients bitwise those of the main-only call, proxy
    # gradients at the same bar
    dout = mi.grad_output(case).cuda()
    main = [torch.full((case.total_q, cfg.hq, 128), float("nan"), device="cuda"),
            torch.full((case.total_k, cfg.hkv, 128), float("nan"), device="cuda"),
            torch.full((case.total_k, cfg.hkv, 128), float("nan"), device="cuda")]
    bws = torch.empty(msa.msa_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    msa.msa_sparse_attn_bwd(s, dev.q, dev.k, dev.v, o, lse, dout, case.softmax_scale, lists_dev,
                            dev.cu_q, dev.cu_k, bws, *main)
    both = [torch.full_like(t, float("nan")) for t in main]
    tws = torch.empty(msa.msa_train_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    tws.fill_(0x3C)
    dqi2, dki2 = torch.full_like(dqi, float("nan")), torch.full_like(dki, float("nan"))
    msa.msa_train_bwd(s, dev.q, dev.k, dev.v, o, lse, dout, case.softmax_scale, dev.q_idx,
                      dev.k_idx, pscale, lists_dev, dev.cu_q, dev.cu_k, tws, *both, dqi2, dki2)
    torch.cuda.synchronize()
    for a_, b_ in zip(main, both):
        assert torch.equal(a_, b_)
    _check("dq_idx (train call)", dqi2.cpu().numpy(), dqi_r)
    _check("dk_idx (train call)", dki2.cpu().numpy(), dki_r)
