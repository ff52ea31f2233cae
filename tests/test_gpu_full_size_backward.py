"""Main-branch backward at the full M3 shape (32K causal, Hq = 64, Hkv = 4, top-16), in the
call sequence a training step runs: index -> forward -> backward.

The oracle cannot differentiate every row in test time, so dQ is compared on a seeded sample
of whole 128-query blocks (rows whose GPU lists equal the oracle's), and dK, dV on properties
that hold at any size: summed over all keys of a group, dV equals the sum of dO over the
group's rows that see a key (each row's weights sum to one) and dK vanishes (each row's dS
sums to zero), up to the bf16 rounding of P, dS and O. A row's weights sum to one within
2^-8 (bf16 rounding of each weight, unbiased), and these row errors are independent, so the
dV sum is held to eight standard deviations, 8 * 2^-8 * sqrt(sum dO^2) per (group, dim),
tight enough that dropping the contributions of one 4096-row chunk (about 64 per dim) fails
it; the dK sum is held to 2e-3 of sum |dK|.
"""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case
from oracle.msa_backward import query_rows_gradient
from synth import msa_inputs as mi
from synth.msa_inputs import widen

from gpu_util import shape_of, upload
from test_gpu_full_size import bench_sequence

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_m3_backward_32k():
    _say("[full-size backward] m3: generating")
    case = mi.make_case("m3", seed=0)
    c = case.cfg
    dev = upload(case)
    chosen, lists, o, lse = bench_sequence(case, dev)
    dout = mi.grad_output(case)
    s = shape_of(case)
    _say("[full-size backward] m3: GPU backward")
    ws = torch.empty(msa.msa_bwd_workspace_size(s), dtype=torch.uint8, device="cuda")
    dq = torch.empty((case.total_q, c.hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((case.total_k, c.hkv, 128), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    msa.msa_sparse_attn_bwd(s, dev.q, dev.k, dev.v, o, lse, dout.cuda(), case.softmax_scale,
                            torch.from_numpy(lists).cuda(), dev.cu_q, dev.cu_k, ws, dq, dk, dv)
    torch.cuda.synchronize()
    del ws, o, lse
    rows = msa_case.sample_rows(case, every=64, seed=0)
    dq_s = dq[torch.from_numpy(rows).cuda()].cpu().numpy()
    dk_n = dk.cpu().numpy().astype(np.float64)
    dv_n = dv.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(dq.cpu().numpy())) and np.all(np.isfinite(dk_n))
    assert np.all(np.isfinite(dv_n))
    del dq, dk, dv, dev
    torch.cuda.empty_cache()

    # dK, dV column sums over every key (one sequence; every row sees its local block)
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

    # dQ on sampled rows, oracle lists; rows whose GPU lists differ (near-ties) are left out
    _say(f"[full-size backward] m3: oracle dQ on {rows.size} rows")
    out = msa_case.run(case, rows=rows, want_output=False)
    same = np.all(lists[rows] == out.topk_idx, axis=(1, 2))
    assert same.mean() > 0.99
    q, k, v = widen(case.q), widen(case.k), widen(case.v)
    want = query_rows_gradient(q, k, v, out.topk_idx[same], do64[rows[same]], rows[same],
                               case.softmax_scale, c.block, c.causal)
    got = dq_s[same]
    d = np.abs(got - want)
    _say(f"  dQ: max |d| {d.max():.3e} (ref max {np.abs(want).max():.3e}), rms "
         f"{np.sqrt(np.mean(d ** 2)):.3e} (ref rms {np.sqrt(np.mean(want ** 2)):.3e}), "
         f"rows {int(same.sum())}")
    assert d.max() <= 2e-2 * np.abs(want).max()
    assert np.sqrt(np.mean(d ** 2)) <= 1e-2 * np.sqrt(np.mean(want ** 2))
