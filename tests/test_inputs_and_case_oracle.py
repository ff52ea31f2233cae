"""Seeded generators (determinism, shapes) and the varlen case driver of the oracle (CPU)."""
import numpy as np
import pytest
import torch

from synth import msa_inputs as mi
from oracle import msa_case, msa_ref as ref
from test_oracle_pins import sdpa


def test_generator_is_thread_count_independent(monkeypatch):
    ss = np.random.SeedSequence(3)
    monkeypatch.setenv("MSA_GEN_THREADS", "1")
    a = mi.normal_f32(ss, (3, mi._CHUNK // 2 + 17))
    monkeypatch.setenv("MSA_GEN_THREADS", "7")
    b = mi.normal_f32(ss, (3, mi._CHUNK // 2 + 17))
    assert np.array_equal(a, b)


def test_cases_are_seeded_and_shaped():
    cfg = mi.custom(n_q=(200, 384), n_k=(300, 384), hq=8, hkv=2, topk=3, dp=16, lowrank=True)
    a, b, c = mi.make_case(cfg, 1), mi.make_case(cfg, 1), mi.make_case(cfg, 2)
    assert torch.equal(a.q, b.q) and torch.equal(a.k_idx, b.k_idx)
    assert not torch.equal(a.q, c.q)
    assert a.q.shape == (584, 8, 128) and a.k.shape == (684, 2, 128)
    assert a.q_idx.shape == (584, 2, 16) and a.k_idx.shape == (684, 2, 16)
    assert list(a.cu_q) == [0, 200, 584] and list(a.cu_k) == [0, 300, 684]


def test_grid_proxies_are_exact_quarters():
    cfg = mi.custom(n_q=(256,), hq=4, hkv=1, proxy="grid", dp=64)
    c = mi.make_case(cfg, 0)
    x = mi.widen(c.q_idx) * 4
    assert np.all(x == np.round(x)) and np.abs(x).max() <= 16


def test_fp8_case_descales():
    cfg = mi.custom(n_q=(128,), hq=4, hkv=1, dtype="fp8")
    c = mi.make_case(cfg, 0)
    assert c.q.dtype == torch.float8_e4m3fn
    qv = mi.widen(c.q, c.descale[0])
    assert abs(np.abs(qv).max() - 448 * c.descale[0]) < 1e-9


def test_decode_lengths():
    c = mi.make_case(mi.Config(name="dec", batch=8, n_q=(), n_k=(), hq=8, hkv=2, topk=4, dp=16,
                               length_seed_draw=(8, 2, 6)), 0)
    nk = np.diff(c.cu_k)
    assert np.all(nk % 128 == 0) and np.all((nk >= 256) & (nk <= 768))
    assert np.all(np.diff(c.cu_q) == 1)


def test_case_oracle_varlen_matches_per_sequence_and_dense():
    cfg = mi.custom(n_q=(200, 256, 1), n_k=(300, 256, 700), hq=4, hkv=2, topk=8, dp=16)
    case = mi.make_case(cfg, 0)
    out = msa_case.run(case)
    assert out.rows.tolist() == list(range(case.total_q))
    # topk covers every block here (nb <= 6 < 8), so each sequence is plain causal attention
    for s in range(3):
        q0, q1 = case.cu_q[s], case.cu_q[s + 1]
        k0, k1 = case.cu_k[s], case.cu_k[s + 1]
        q = mi.widen(case.q)[q0:q1]
        k = mi.widen(case.k)[k0:k1]
        v = mi.widen(case.v)[k0:k1]
        n_q, n_k = q1 - q0, k1 - k0
        mask = np.arange(n_k)[None, :] <= (n_k - n_q) + np.arange(n_q)[:, None]
        np.testing.assert_allclose(out.o[q0:q1], sdpa(q, k, v, mask, case.softmax_scale), atol=1e-12)


def test_case_oracle_row_sampling_is_consistent():
    cfg = mi.custom(n_q=(640,), hq=4, hkv=2, topk=3, dp=16, lowrank=True)
    case = mi.make_case(cfg, 0)
    full = msa_case.run(case)
    rows = msa_case.sample_rows(case, every=2, seed=1)
    part = msa_case.run(case, rows=rows)
    assert np.array_equal(part.topk_idx, full.topk_idx[rows])
    np.testing.assert_allclose(part.o, full.o[rows], atol=0)


def test_case_oracle_tile_lists():
    cfg = mi.custom(n_q=(384,), n_k=(1024,), hq=2, hkv=2, topk=3, causal=False, list_q=128,
                    list_pool=8)
    case = mi.make_case(cfg, 0)
    assert case.lists.shape == (3, 2, 3)
    out = msa_case.run(case)
    q, k, v = mi.widen(case.q), mi.widen(case.k), mi.widen(case.v)
    for t in range(3):
        for h in range(2):
            keys = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in case.lists[t, h]])
            qq = q[t * 128:(t + 1) * 128, h:h + 1]
            e = sdpa(qq, k[keys, h:h + 1], v[keys, h:h + 1], np.ones((128, keys.size), bool),
                     case.softmax_scale)
            np.testing.assert_allclose(out.o[t * 128:(t + 1) * 128, h:h + 1], e, atol=1e-12)


def test_fp8_proxies_from_the_same_draws_and_scale_invariant():
    """e4m3 proxies: codes within +-448 with descale amax / 448, drawn from the same numbers as
    the bf16 proxies of the same seed; the oracle's selection on the dequantised proxies is
    the selection on the codes alone (a positive factor keeps the order) and its block scores
    are the codes' scores times the two descales."""
    kw = dict(n_q=(300,), n_k=(700,), hq=4, hkv=2, topk=5, dp=32)
    case = mi.make_case(mi.custom(name="p8", idx_dtype="fp8", **kw), seed=3)
    bf = mi.make_case(mi.custom(name="p8", **kw), seed=3)
    assert case.q_idx.dtype == torch.float8_e4m3fn and case.k_idx.dtype == torch.float8_e4m3fn
    dqi, dki = case.idx_descale
    for t8, t16, d in ((case.q_idx, bf.q_idx, dqi), (case.k_idx, bf.k_idx, dki)):
        c = mi.widen(t8)
        assert np.max(np.abs(c)) == 448.0                 # amax maps to the largest code
        a8, a16 = c * d, mi.widen(t16)
        # e4m3 keeps 3 fraction bits (subnormal step 2^-9 x descale), bf16 7
        assert np.all(np.abs(a8 - a16) <= 2.0 ** -4 * np.abs(a16) + 2.0 ** -9 * d)
    out = msa_case.run(case, want_output=False)
    case.idx_descale = (1.0, 1.0)
    out1 = msa_case.run(case, want_output=False)
    assert np.array_equal(out.topk_idx, out1.topk_idx)
    fin = np.isfinite(out1.scores[0])
    assert np.array_equal(np.isfinite(out.scores[0]), fin)
    np.testing.assert_allclose(out.scores[0][fin], out1.scores[0][fin] * dqi * dki, rtol=1e-12)
