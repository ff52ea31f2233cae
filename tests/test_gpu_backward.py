"""Main-branch backward on the GPU (libmsa through its C ABI) against the fp64 oracle.

Both sides take the same block lists (the oracle's own index branch, or the case's per-tile
lists) and the same bf16 Q, K, V, dO. The GPU backward consumes the GPU forward's bf16 O and
fp32 LSE, as a training step would; the oracle recomputes both in fp64.

Bar, derived from the arithmetic: P and dS enter the MFMA products rounded to bf16 (relative
2^-9 each), O enters D = dO.O rounded to bf16, and the forward's LSE carries its own fp32
error; each gradient element is a sum of such products over at most topk * 128 keys (dQ) or
the queries that chose a block (dK, dV), accumulated in fp32. Per tensor:
max |G - G_ref| <= 2e-2 * max |G_ref| and rms(G - G_ref) <= 1e-2 * rms(G_ref).
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_backward
from synth import msa_inputs as mi

from gpu_util import shape_of, upload

pytestmark = pytest.mark.gpu

MAX_REL, RMS_REL = 2e-2, 1e-2

CASES = [
    # G = 16, one sequence spanning several blocks and query ranges, causal
    ("g16_causal", dict(n_q=(700,), n_k=(700,), hq=16, hkv=1, topk=4)),
    # G = 4, ragged varlen with a single-query sequence and a short one
    ("g4_ragged", dict(n_q=(300, 1, 129), n_k=(700, 4000, 129), hq=8, hkv=2, topk=5)),
    # G = 1, non-causal
    ("g1_noncausal", dict(n_q=(200, 384), n_k=(1000, 384), hq=2, hkv=2, topk=6, causal=False)),
    # G = 2 and G = 8
    ("g2", dict(n_q=(520,), n_k=(1300,), hq=4, hkv=2, topk=3)),
    ("g8_decode", dict(n_q=(1, 2, 3), n_k=(4096 + 77, 256, 130), hq=16, hkv=2, topk=8)),
    # every query selects every block: columns of 4500 entries split into two chunks of 4096
    # rows whose dK / dV partials are summed (G = 1), and many chunks per column at G = 16
    ("g1_split_columns", dict(n_q=(4500,), n_k=(600,), hq=1, hkv=1, topk=5, causal=False)),
    ("g16_split_columns", dict(n_q=(1100,), n_k=(512,), hq=16, hkv=1, topk=4, causal=False)),
    # per-Q-tile lists (list_q = 128) drawn by the case
    ("g8_tile_lists", dict(n_q=(384, 200), n_k=(1024, 640), hq=8, hkv=1, topk=4, list_q=128,
                           list_pool=8)),
]


def _say(*a):
    print(*a, flush=True)


def _gpu_backward(case, dev, lists_dev, list_q, dout):
    s = shape_of(case, list_q)
    ws_f = torch.zeros(msa.msa_workspace_size(s, msa.MSA_KV_OUTER), dtype=torch.uint8,
                       device="cuda")
    o = torch.empty((case.total_q, case.cfg.hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.total_q, case.cfg.hq), dtype=torch.float32, device="cuda")
    msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, None, case.softmax_scale, lists_dev,
                            dev.cu_q, dev.cu_k, msa.MSA_KV_OUTER, ws_f, o, lse)
    msa.msa_combine(s, msa.MSA_KV_OUTER, ws_f, o, lse)
    ws = torch.empty(msa.msa_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5)                       # the call must not depend on a cleared workspace
    dq = torch.full((case.total_q, case.cfg.hq, 128), float("nan"), device="cuda")
    dk = torch.full((case.total_k, case.cfg.hkv, 128), float("nan"), device="cuda")
    dv = torch.full_like(dk, float("nan"))
    msa.msa_sparse_attn_bwd(s, dev.q, dev.k, dev.v, o, lse, dout.to("cuda"), case.softmax_scale,
                            lists_dev, dev.cu_q, dev.cu_k, ws, dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _check(name, got, want):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - want)
    ref_max = float(np.abs(want).max()) if want.size else 0.0
    ref_rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    mx = float(d.max()) if d.size else 0.0
    rms = float(np.sqrt(np.mean(d ** 2))) if d.size else 0.0
    _say(f"  {name}: max |d| {mx:.3e} (ref max {ref_max:.3e}), rms {rms:.3e} "
         f"(ref rms {ref_rms:.3e})")
    assert mx <= MAX_REL * ref_max + 1e-6, name
    assert rms <= RMS_REL * ref_rms + 1e-7, name


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, kw):
    cfg = mi.custom(name, **kw)
    case = mi.make_case(cfg, seed=11)
    dout = mi.grad_output(case)
    _say(f"[backward] {name}: total_q {case.total_q} total_k {case.total_k} "
         f"hq {cfg.hq} hkv {cfg.hkv} topk {cfg.topk} list_q {cfg.list_q}")
    dq_r, dk_r, dv_r, _, _, lists = msa_backward.run_case(case, dout)
    dev = upload(case)
    if cfg.list_q == 1:
        lists_dev, list_q = torch.from_numpy(lists).to("cuda"), 1
    else:
        lists_dev, list_q = dev.lists, cfg.list_q
    dq, dk, dv = _gpu_backward(case, dev, lists_dev, list_q, dout)
    _check("dQ", dq, dq_r)
    _check("dK", dk, dk_r)
    _check("dV", dv, dv_r)


def test_backward_no_queries_and_unselected_keys():
    """Keys no query selects get zero gradients; a sequence with no queries leaves its keys at
    zero; query rows with no visible key (an empty list) get dQ = 0."""
    cfg = mi.custom("bwd_edges", n_q=(0, 64), n_k=(512, 1024), hq=4, hkv=1, topk=2)
    case = mi.make_case(cfg, seed=5)
    dout = mi.grad_output(case)
    lists = np.full((case.total_q, 1, 2), -1, dtype=np.int32)
    lists[:32, 0, 0] = 7                 # the local block of the 64 queries of sequence 1
    dq_r, dk_r, dv_r, _, _, _ = msa_backward.run_case(case, dout, lists=lists)
    dev = upload(case)
    dq, dk, dv = _gpu_backward(case, dev, torch.from_numpy(lists).to("cuda"), 1, dout)
    assert np.all(dq[32:] == 0) and np.all(dk[:512 + 896] == 0) and np.all(dv[:512 + 896] == 0)
    _check("dQ", dq, dq_r)
    _check("dK", dk, dk_r)
    _check("dV", dv, dv_r)
