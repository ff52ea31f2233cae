"""Helpers for the GPU tests: upload a seeded case, run the library, compare with the oracle."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from block_sparse_gqa_amd import msa
from synth.msa_inputs import Case


@dataclass
class Dev:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_idx: torch.Tensor | None
    k_idx: torch.Tensor | None
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    lists: torch.Tensor | None
    descale: torch.Tensor | None
    idx_descale: torch.Tensor | None = None   # fp8 proxies: device [descale q_idx, k_idx]


def upload(case: Case, device="cuda") -> Dev:
    def up(t):
        return None if t is None else t.contiguous().to(device)
    lists = None if case.lists is None else torch.from_numpy(case.lists).to(device)
    ds = None
    if case.cfg.dtype == "fp8":
        ds = torch.tensor(case.descale, dtype=torch.float32, device=device)
    ids = None
    if case.cfg.idx_dtype == "fp8":
        ids = torch.tensor(case.idx_descale, dtype=torch.float32, device=device)
    return Dev(q=up(case.q), k=up(case.k), v=up(case.v), q_idx=up(case.q_idx),
               k_idx=up(case.k_idx), cu_q=torch.from_numpy(case.cu_q).to(device),
               cu_k=torch.from_numpy(case.cu_k).to(device), lists=lists, descale=ds,
               idx_descale=ids)


def shape_of(case: Case, list_q=None) -> msa.Shape:
    c = case.cfg
    return msa.make_shape(batch=len(case.cu_q) - 1, total_q=case.total_q, total_k=case.total_k,
                          max_q=case.max_q, max_k=case.max_k, hq=c.hq, hkv=c.hkv, topk=c.topk,
                          dp=c.dp, causal=c.causal,
                          dtype=msa.MSA_FP8_E4M3 if c.dtype == "fp8" else msa.MSA_BF16,
                          list_q=c.list_q if list_q is None else list_q)


def run_index(case: Case, dev: Dev, s, topk, score, ws) -> None:
    """The index branch for the case's proxy type (bf16, or fp8 with its descales)."""
    if case.cfg.idx_dtype == "fp8":
        msa.msa_index_topk_fp8(s, dev.q_idx, dev.k_idx, dev.idx_descale, dev.cu_q, dev.cu_k,
                               topk, score, ws)
    else:
        msa.msa_index_topk(s, dev.q_idx, dev.k_idx, dev.cu_q, dev.cu_k, topk, score, ws)


def proxies(case: Case) -> tuple[np.ndarray, np.ndarray]:
    """The proxies' exact values as float64 (fp8 codes times their descales)."""
    from synth.msa_inputs import widen
    dqi, dki = case.idx_descale
    return widen(case.q_idx, dqi), widen(case.k_idx, dki)


def gpu_index(case: Case, dev: Dev):
    s = shape_of(case)
    topk = torch.full((case.total_q, case.cfg.hkv, case.cfg.topk), -7, dtype=torch.int32,
                      device="cuda")
    score = torch.full(topk.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(msa.msa_index_workspace_size(s), 256), dtype=torch.uint8, device="cuda")
    run_index(case, dev, s, topk, score, ws)
    torch.cuda.synchronize()
    return topk.cpu().numpy(), score.cpu().numpy()


def gpu_attention(case: Case, dev: Dev, lists: torch.Tensor, mode: int, list_q=None,
                  keep_ws=False):
    s = shape_of(case, list_q)
    chosen = msa.msa_resolve_mode(s, mode)
    ws = torch.zeros(msa.msa_workspace_size(s, chosen), dtype=torch.uint8, device="cuda")
    o = torch.full((case.total_q, case.cfg.hq, 128), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    lse = torch.full((case.total_q, case.cfg.hq), float("nan"), dtype=torch.float32,
                     device="cuda")
    msa.msa_sparse_attn_fwd(s, dev.q, dev.k, dev.v, dev.descale, case.softmax_scale, lists,
                            dev.cu_q, dev.cu_k, chosen, ws, o, lse)
    msa.msa_combine(s, chosen, ws, o, lse)
    torch.cuda.synchronize()
    out = (o.float().cpu().numpy(), lse.cpu().numpy())
    if keep_ws:
        return out + (ws, s, chosen)
    return out


# Error of one e4m3 proxy dot product on the 8-bit MFMA, relative to sum_d |q_d k_d|: the
# products are summed in aligned groups of 8, each aligned to its largest product's exponent E
# with the bits below 2^(E - 13) dropped (measured on the MI355X: of 448 + 63 x 2^-s, the 7
# small terms sharing the large term's group vanish for s >= 6 and stay for s <= 5), so each
# of the 7 other products of a group loses less than 2^-13 of the group's largest; the 8
# group sums and the descale product add fp32 roundings.
FP8_DOT_REL = 7 * 2.0 ** -13 + 10 * 2.0 ** -24


def near_tie_bound(qi: np.ndarray, ki: np.ndarray, fp8: bool = False) -> float:
    """Twice the error bound of one proxy dot product for one (query, group), as a multiple of
    |q|_2 * max_u |k_u|_2 >= sum_d |q_d k_ud|: bf16 proxies, fp32 summation gamma_dp (Higham);
    fp8 proxies, FP8_DOT_REL."""
    dp = qi.shape[-1]
    gamma = FP8_DOT_REL if fp8 else dp * 2.0 ** -24 / (1 - dp * 2.0 ** -24)
    return 2 * gamma * float(np.linalg.norm(qi)) * float(np.max(np.linalg.norm(ki, axis=-1)))


def compare_lists(gpu: np.ndarray, ref: np.ndarray, scores_ref, bound_fn=None):
    """Bit-exact list comparison; with ``bound_fn`` (row, group) -> bound, rows whose lists
    differ only by swaps between blocks whose fp64 proxy scores are within the bound are
    counted as certified near-ties. Returns (n_exact_mismatch_rows, n_near_tie_rows, bad)."""
    diff_rows = np.nonzero(np.any(gpu != ref, axis=2))
    n_tie, bad = 0, []
    for i, g in zip(*diff_rows):
        if bound_fn is None:
            bad.append((int(i), int(g)))
            continue
        sc = scores_ref(i, g)
        bd = bound_fn(i, g)
        a = [b for b in ref[i, g] if b >= 0]
        b_ = [b for b in gpu[i, g] if b >= 0]
        ok = len(a) == len(b_) and a[0] == b_[0]
        # same multiset of scores up to the bound, position by position
        if ok:
            for x, y in zip(a, b_):
                if abs(sc[x] - sc[y]) > bd and not (np.isinf(sc[x]) and sc[x] == sc[y]):
                    ok = False
                    break
        if ok:
            n_tie += 1
        else:
            bad.append((int(i), int(g)))
    return len(diff_rows[0]), n_tie, bad


def err_stats(o_gpu, o_ref, lse_gpu, lse_ref):
    fin = np.isfinite(lse_ref)
    d = np.abs(o_gpu - o_ref)
    dl = np.abs(np.where(fin, lse_gpu - lse_ref, 0.0))
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "rel_rms": float(math.sqrt(np.mean(d ** 2) / max(np.mean(o_ref ** 2), 1e-30))) if d.size else 0.0,
        "max_dlse": float(dl.max()) if dl.size else 0.0,
        "lse_inf_match": bool(np.all(np.isneginf(lse_gpu[~fin]))) if (~fin).any() else True,
    }
