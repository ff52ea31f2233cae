"""Whole-layer oracle over a seeded varlen input set (TEST INFRASTRUCTURE ONLY).

Widens the stored bf16/fp8 inputs to their exact fp64 values (fp8 codes times their
per-tensor descale) and runs the fp64 definition of ``msa_ref`` sequence by sequence:
index branch for the sampled query rows, then exact sparse attention for the same rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from synth.msa_inputs import Case, widen
from . import msa_ref as ref
from . import mxfp4


@dataclass
class OracleOut:
    rows: np.ndarray          # global query token indices covered
    topk_idx: np.ndarray      # [n, Hkv, K] int32 (per-query lists; expanded for tile lists)
    scores: list              # per sequence: proxy block scores [n_s, Hkv, nb_s] (None for given lists)
    o: np.ndarray             # [n, Hq, D] fp64
    lse: np.ndarray           # [n, Hq] fp64


def seq_rows(case: Case, rows: np.ndarray | None):
    """Split global query rows by sequence: yields (s, q0, q1, k0, k1, local_rows)."""
    for s in range(len(case.cu_q) - 1):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        k0, k1 = int(case.cu_k[s]), int(case.cu_k[s + 1])
        if rows is None:
            loc = np.arange(q1 - q0)
        else:
            r = np.asarray(rows)
            loc = r[(r >= q0) & (r < q1)] - q0
        yield s, q0, q1, k0, k1, loc


def tile_base(case: Case, s: int) -> int:
    """Row of sequence s's first tile list: lists are laid out [B * tiles_max, Hkv, K]."""
    tiles_max = -(-case.max_q // case.cfg.list_q)
    return s * tiles_max


def run(case: Case, rows: np.ndarray | None = None, lists: np.ndarray | None = None,
        want_output: bool = True) -> OracleOut:
    """Oracle forward of ``case`` on global query ``rows`` (default: all queries).

    ``lists``: per-query block lists [Tq, Hkv, K] to use instead of the index branch (for
    checking the main branch on the lists another path selected). Given per-tile lists of
    the case (list_q > 1) are used when the case has them."""
    cfg = case.cfg
    dq, dk, dv = case.descale
    q = widen(case.q, dq)
    k = widen(case.k, dk)
    v = widen(case.v, dv)
    # proxies: bf16, or e4m3 codes times their per-tensor descale ("Sparse Attention",
    # Chapter 4: the low-precision scorer compares quantised index vectors; the selection rule
    # is unchanged)
    dqi, dki = case.idx_descale
    if cfg.idx_dtype == "mxfp4":
        # 4-bit codes times their E8M0 group scales ("Sparse Attention", Chapter 4, FP4)
        qi = mxfp4.dequantize(case.q_idx.numpy(), case.q_idx_scale.numpy())
        ki = mxfp4.dequantize(case.k_idx.numpy(), case.k_idx_scale.numpy())
    else:
        qi = widen(case.q_idx, dqi) if case.q_idx is not None else None
        ki = widen(case.k_idx, dki) if case.k_idx is not None else None
    out_rows, out_sel, out_s, out_o, out_l = [], [], [], [], []
    for s, q0, q1, k0, k1, loc in seq_rows(case, rows):
        if loc.size == 0:
            continue
        n_q = q1 - q0
        if lists is not None:
            sel_full = None
            sel = lists[q0 + loc]
            sc = None
        elif case.lists is not None:
            base = tile_base(case, s)
            sel = case.lists[base + loc // cfg.list_q]
            sc = None
        else:
            sel, sc = ref.index_topk(qi[q0:q1], ki[k0:k1], cfg.block, cfg.topk, cfg.causal,
                                     rows=loc)
        out_rows.append(q0 + loc)
        out_sel.append(sel)
        out_s.append(sc)
        if want_output:
            # sparse_attention indexes lists by query row: scatter the rows' lists in place
            full = np.full((n_q, cfg.hkv, sel.shape[2]), -1, dtype=np.int32)
            full[loc] = sel
            o, l = ref.sparse_attention(q[q0:q1], k[k0:k1], v[k0:k1], full, case.softmax_scale,
                                        cfg.block, cfg.causal, rows=loc)
            out_o.append(o)
            out_l.append(l)
    cat = (lambda xs: np.concatenate(xs, axis=0)) if out_rows else (lambda xs: None)
    return OracleOut(rows=cat(out_rows), topk_idx=cat(out_sel), scores=out_s,
                     o=cat(out_o) if want_output and out_o else None,
                     lse=cat(out_l) if want_output and out_l else None)


def sample_rows(case: Case, every: int = 16, seed: int = 0, block: int = 128) -> np.ndarray:
    """Systematic sample of whole query blocks: every ``every``-th 128-query block of each
    sequence, starting at a seeded offset (all rows of each sampled block)."""
    rng = np.random.default_rng(seed)
    off = int(rng.integers(0, every))
    out = []
    for s in range(len(case.cu_q) - 1):
        q0, q1 = int(case.cu_q[s]), int(case.cu_q[s + 1])
        nqb = -(-(q1 - q0) // block)
        for b in range(off % max(1, min(every, nqb)), nqb, every):
            out.append(np.arange(q0 + b * block, min(q1, q0 + (b + 1) * block)))
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)
