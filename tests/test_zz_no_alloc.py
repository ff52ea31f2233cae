"""The allocation-free main-branch call (msa_sparse_attn_fwd_noalloc, scratch held by the
library) against the workspace form (msa_sparse_attn_fwd + msa_combine on a caller-allocated
workspace) through the C ABI: the same kernels run, so outputs must be bitwise equal. Two calls
in a row on the library's scratch, the second with a smaller input, for each schedule; a shape
whose workspace exceeds the scratch is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

from block_sparse_gqa_amd import msa
from oracle import msa_case
from synth import msa_inputs as mi

from gpu_util import gpu_attention, shape_of, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _noalloc(case, dev, lists, mode):
    s = shape_of(case)
    o = torch.full((case.total_q, case.cfg.hq, 128), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    lse = torch.full((case.total_q, case.cfg.hq), float("nan"), dtype=torch.float32,
                     device="cuda")
    msa.msa_sparse_attn_fwd_noalloc(s, dev.q, dev.k, dev.v, dev.descale, case.softmax_scale,
                                    lists, dev.cu_q, dev.cu_k, mode, o, lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


CASES = [
    # (schedule, larger case, smaller case)
    ("kv_outer", msa.MSA_KV_OUTER,
     mi.custom(name="na1", n_q=(2048,), hq=16, hkv=1, topk=4, dp=32),
     mi.custom(name="na2", n_q=(300, 200), n_k=(700, 200), hq=8, hkv=2, topk=5, dp=32)),
    ("kv_outer_fp8", msa.MSA_KV_OUTER,
     mi.custom(name="na3", n_q=(1024,), hq=16, hkv=2, topk=6, dp=32, dtype="fp8"),
     mi.custom(name="na4", n_q=(256,), hq=4, hkv=2, topk=3, dp=32, dtype="fp8")),
    ("q_outer_decode", msa.MSA_AUTO,
     mi.Config(name="na5", batch=8, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
               length_seed_draw=(8, 16, 64)),
     mi.Config(name="na6", batch=3, n_q=(), n_k=(), hq=64, hkv=4, topk=16, dp=64,
               length_seed_draw=(3, 16, 40))),
]


@pytest.mark.parametrize("name,mode,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_the_workspace_call(name, mode, big, small):
    for tag, cfg in (("first call", big), ("second call, smaller", small)):
        case = mi.make_case(cfg, seed=3)
        dev = upload(case)
        lists = torch.from_numpy(msa_case.run(case, want_output=False).topk_idx).cuda()
        s = shape_of(case)
        need = msa.msa_workspace_size(s, msa.msa_resolve_mode(s, mode))
        _say(f"[noalloc] {name} {tag}: total_q {case.total_q}, scratch {need} bytes")
        assert need <= (64 << 20)
        o_ref, l_ref = gpu_attention(case, dev, lists, mode)
        o, l = _noalloc(case, dev, lists, mode)
        assert np.array_equal(o, o_ref), float(np.nanmax(np.abs(o - o_ref)))
        assert np.array_equal(l, l_ref, equal_nan=True)


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    """Valid, in-bounds inputs of a shape whose workspace exceeds the scratch: the call is
    rejected on the host and the outputs stay untouched."""
    n, hq, hkv, k = 16384, 64, 4, 16
    s = msa.make_shape(batch=1, total_q=n, total_k=n, max_q=n, max_k=n, hq=hq, hkv=hkv, topk=k,
                       dp=64)
    assert msa.msa_workspace_size(s, msa.MSA_KV_OUTER) > (64 << 20)
    q = torch.zeros((n, hq, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((n, hkv, 128), dtype=torch.bfloat16, device="cuda")
    lists = torch.full((n, hkv, k), -1, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    o = torch.full((n, hq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((n, hq), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(msa.MSAError) as ei:
        msa.msa_sparse_attn_fwd_noalloc(s, q, kv, kv, None, 0.1, lists, cu, cu,
                                        msa.MSA_KV_OUTER, o, lse)
    assert ei.value.status == msa.MSA_ERR_WORKSPACE and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0)) and bool(torch.all(lse == 7.0))
