"""Host side of libmsa's C ABI, with no GPU: the library loads, exports every function that
include/msa.h declares, validates arguments before anything is enqueued, sizes its
workspace as documented, and applies the schedule rule and the crossover model.

Nothing here launches a kernel: every device entry point is called with arguments that the
host checks reject, so the calls return before touching the HIP runtime.
"""
import ctypes
import json
import os
import re

import pytest

from block_sparse_gqa_amd import msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_figures.json")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(msa.LIB_PATH):
        from block_sparse_gqa_amd import build
        build.build()
    return msa.lib()


def m3_shape(**kw):
    base = dict(batch=1, total_q=32768, total_k=32768, max_q=32768, max_k=32768, hq=64, hkv=4,
                topk=16, dp=64)
    base.update(kw)
    return msa.make_shape(**base)


def decode_shape():
    # 64 requests of one query each over KV caches of up to 131072 keys
    return msa.make_shape(batch=64, total_q=64, total_k=64 * 70000, max_q=1, max_k=131072,
                          hq=64, hkv=4, topk=16, dp=64)


# ------------------------------------------------------------------ symbols


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(msa.SYMBOLS)


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings(L):
    seen = set()
    for st in range(7):
        s = msa.lib().msa_status_string(st).decode()
        assert s and s not in seen
        seen.add(s)
    assert msa.lib().msa_status_string(99).decode() == "unknown status"


# ------------------------------------------------------------------ shape checks

BAD_SHAPES = [
    ("d", dict(d=64), msa.MSA_ERR_SHAPE),
    ("block", dict(block=64), msa.MSA_ERR_SHAPE),
    ("topk0", dict(topk=0), msa.MSA_ERR_SHAPE),
    ("topk17", dict(topk=17), msa.MSA_ERR_SHAPE),
    ("group3", dict(hq=12, hkv=4), msa.MSA_ERR_SHAPE),
    ("group32", dict(hq=64, hkv=2), msa.MSA_ERR_SHAPE),
    ("hq_not_multiple", dict(hq=10, hkv=4), msa.MSA_ERR_SHAPE),
    ("list_q", dict(list_q=64), msa.MSA_ERR_SHAPE),
    ("causal", dict(causal=2), msa.MSA_ERR_SHAPE),
    ("max_q_gt_total", dict(max_q=40000), msa.MSA_ERR_SHAPE),
    ("negative", dict(total_k=-1), msa.MSA_ERR_SHAPE),
    ("batch0", dict(batch=0), msa.MSA_ERR_SHAPE),
    ("dtype", dict(dtype=7), msa.MSA_ERR_DTYPE),
    ("int32_entries", dict(total_q=1 << 24, max_q=1 << 24, total_k=1 << 24, max_k=1 << 24),
     msa.MSA_ERR_SHAPE),
]


@pytest.mark.parametrize("name,kw,status", BAD_SHAPES, ids=[b[0] for b in BAD_SHAPES])
def test_bad_shapes_are_rejected_by_every_entry_point(L, name, kw, status):
    s = m3_shape(**kw)
    if name == "causal":
        s.causal = 2
    n = ctypes.c_size_t(0)
    assert L.msa_workspace_size(ctypes.byref(s), msa.MSA_AUTO, ctypes.byref(n)) == status
    m = ctypes.c_int(0)
    assert L.msa_resolve_mode(ctypes.byref(s), msa.MSA_AUTO, ctypes.byref(m)) == status
    # device entry points: rejected before any launch
    fake = ctypes.c_void_p(0x1000)
    assert L.msa_index_topk(ctypes.byref(s), fake, fake, fake, fake, fake, None, None, 0,
                            None) == status
    assert L.msa_index_topk_fp8(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, None,
                                0, None) == status
    assert L.msa_select_tiles(ctypes.byref(s), 4, fake, fake, fake, fake, fake, None, fake,
                              1 << 40, None) == status
    assert L.msa_select_workspace_size(ctypes.byref(s), 4, ctypes.byref(n)) == status
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, fake, fake, None, 0.1, fake, fake, fake,
                                 msa.MSA_AUTO, fake, 1 << 40, fake, None, None) == status
    assert L.msa_combine(ctypes.byref(s), msa.MSA_AUTO, fake, 1 << 40, fake, None,
                         None) == status


def test_null_shape_and_outputs(L):
    n = ctypes.c_size_t(0)
    assert L.msa_workspace_size(None, msa.MSA_AUTO, ctypes.byref(n)) == msa.MSA_ERR_NULL
    s = m3_shape()
    assert L.msa_workspace_size(ctypes.byref(s), msa.MSA_AUTO, None) == msa.MSA_ERR_NULL
    assert L.msa_resolve_mode(ctypes.byref(s), msa.MSA_AUTO, None) == msa.MSA_ERR_NULL
    assert L.msa_crossover(ctypes.byref(s), 8.0, 16.0, None) == msa.MSA_ERR_NULL


def test_null_device_pointers_and_small_workspace(L):
    s = m3_shape()
    fake = ctypes.c_void_p(0x1000)
    need = msa.msa_workspace_size(s, msa.MSA_AUTO)
    # index branch: missing lists / inputs
    assert L.msa_index_topk(ctypes.byref(s), fake, fake, fake, fake, None, None, None, 0,
                            None) == msa.MSA_ERR_NULL
    assert L.msa_index_topk(ctypes.byref(s), None, fake, fake, fake, fake, None, None, 0,
                            None) == msa.MSA_ERR_NULL
    # unsupported proxy width
    s_dp = m3_shape(dp=48)
    assert L.msa_index_topk(ctypes.byref(s_dp), fake, fake, fake, fake, fake, None, None, 0,
                            None) == msa.MSA_ERR_SHAPE
    # fp8 proxies: the descales are required
    assert L.msa_index_topk_fp8(ctypes.byref(s), fake, fake, None, fake, fake, fake, None, None,
                                0, None) == msa.MSA_ERR_NULL
    assert L.msa_index_topk_fp8(ctypes.byref(s_dp), fake, fake, fake, fake, fake, fake, None,
                                None, 0, None) == msa.MSA_ERR_SHAPE
    # MXFP4 proxies: both scale arrays are required, dp as for the other precisions
    assert L.msa_index_topk_mxfp4(ctypes.byref(s), fake, None, fake, fake, fake, fake, fake,
                                  None, None, 0, None) == msa.MSA_ERR_NULL
    assert L.msa_index_topk_mxfp4(ctypes.byref(s), fake, fake, fake, None, fake, fake, fake,
                                  None, None, 0, None) == msa.MSA_ERR_NULL
    assert L.msa_index_topk_mxfp4(ctypes.byref(s_dp), fake, fake, fake, fake, fake, fake, fake,
                                  None, None, 0, None) == msa.MSA_ERR_SHAPE
    # main branch: workspace checks come first, then pointers
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, fake, fake, None, 0.1, fake, fake, fake,
                                 msa.MSA_AUTO, fake, need - 1, fake, None,
                                 None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, fake, fake, None, 0.1, fake, fake, fake,
                                 msa.MSA_AUTO, None, need, fake, None,
                                 None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, None, fake, None, 0.1, fake, fake, fake,
                                 msa.MSA_AUTO, fake, need, fake, None,
                                 None) == msa.MSA_ERR_NULL
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, fake, fake, None, 0.1, None, fake, fake,
                                 msa.MSA_AUTO, fake, need, fake, None,
                                 None) == msa.MSA_ERR_NULL
    s8 = m3_shape(dtype=msa.MSA_FP8_E4M3)
    need8 = msa.msa_workspace_size(s8, msa.MSA_AUTO)
    assert L.msa_sparse_attn_fwd(ctypes.byref(s8), fake, fake, fake, None, 0.1, fake, fake, fake,
                                 msa.MSA_AUTO, fake, need8, fake, None,
                                 None) == msa.MSA_ERR_NULL
    assert L.msa_combine(ctypes.byref(s), msa.MSA_AUTO, fake, need, None, None,
                         None) == msa.MSA_ERR_NULL
    assert L.msa_combine(ctypes.byref(s), msa.MSA_AUTO, fake, need - 1, fake, None,
                         None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_plan(ctypes.byref(s), None, fake, fake, fake, need, None) == msa.MSA_ERR_NULL
    assert L.msa_attn_main(ctypes.byref(s), fake, fake, fake, None, 0.1, fake, fake, fake, 16,
                           None) == msa.MSA_ERR_WORKSPACE
    # a mode outside the enum
    assert L.msa_sparse_attn_fwd(ctypes.byref(s), fake, fake, fake, None, 0.1, fake, fake, fake,
                                 5, fake, need, fake, None, None) == msa.MSA_ERR_MODE


def test_selector_argument_checks(L):
    """Per-tile lists only, bf16 Q/K only, one or four representatives, pointers and
    workspace checked before any launch."""
    fake = ctypes.c_void_p(0x1000)
    s = msa.make_shape(batch=2, total_q=8192, total_k=32768, max_q=4096, max_k=16384, hq=16,
                       hkv=1, topk=16, causal=False, list_q=128)
    need = msa.msa_select_workspace_size(s, 4)
    # representatives (fp32) of 64 tiles x 16 heads and 256 blocks, 4 each, and the scores
    assert need >= 64 * 16 * 4 * 128 * 4 + 256 * 4 * 128 * 4 + 64 * 128 * 4
    assert msa.msa_select_workspace_size(s, 1) < need
    sel = lambda shape, reps, ws=fake, nbytes=need, lists=fake, q=fake: L.msa_select_tiles(
        ctypes.byref(shape), reps, q, fake, fake, fake, lists, None, ws, nbytes, None)
    assert sel(s, 2) == msa.MSA_ERR_SHAPE
    assert sel(msa.make_shape(batch=2, total_q=8192, total_k=32768, max_q=4096, max_k=16384,
                              hq=16, hkv=1, topk=16, causal=False), 4) == msa.MSA_ERR_SHAPE
    s8 = msa.make_shape(batch=2, total_q=8192, total_k=32768, max_q=4096, max_k=16384, hq=16,
                        hkv=1, topk=16, causal=False, list_q=128, dtype=msa.MSA_FP8_E4M3)
    assert sel(s8, 4) == msa.MSA_ERR_DTYPE
    assert sel(s, 4, lists=None) == msa.MSA_ERR_NULL
    assert sel(s, 4, q=None) == msa.MSA_ERR_NULL
    assert sel(s, 4, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE
    assert sel(s, 4, ws=None) == msa.MSA_ERR_WORKSPACE


def test_python_binding_raises_on_error(L):
    with pytest.raises(msa.MSAError) as ei:
        msa.msa_workspace_size(m3_shape(d=64), msa.MSA_AUTO)
    assert ei.value.status == msa.MSA_ERR_SHAPE


# ------------------------------------------------------------------ workspace layout


def test_kv_outer_workspace_layout_m3():
    s = m3_shape()
    lay = msa.msa_workspace_layout_of(s, msa.MSA_KV_OUTER)
    e_max = 32768 * 4 * 16
    G = 16
    regions = [lay.counters, lay.masks, lay.offsets, lay.scan_sums, lay.entry_q,
               lay.entry_bucket, lay.cmap, lay.part_lse, lay.part_l, lay.part_o]
    assert regions == sorted(regions) and all(r % 256 == 0 for r in regions)
    assert lay.part_l - lay.part_lse >= e_max * G * 4
    assert lay.part_o - lay.part_l >= e_max * G * 4
    assert lay.total - lay.part_o >= e_max * G * 128 * 2
    assert lay.slots == 16 and lay.nb_max == 256
    assert lay.n_words == lay.words_per_bucket * lay.n_ranges * 4 * lay.nb_max
    assert msa.msa_workspace_size(s, msa.MSA_KV_OUTER) == lay.total


def test_kv_outer_workspace_holds_the_transposed_v():
    """KV-outer, bf16 and fp8 alike: a bf16 V^T of every (group, key block) before the partials,
    hkv * (ceil(total_k / 128) + batch) blocks of 128 x 128 elements (the blocks of each
    sequence numbered from its first key); Q-outer: no such region."""
    for s in (m3_shape(), m3_shape(dtype=msa.MSA_FP8_E4M3)):
        lay = msa.msa_workspace_layout_of(s, msa.MSA_KV_OUTER)
        assert lay.cmap < lay.v_wide < lay.part_lse and lay.v_wide % 256 == 0
        need = 4 * (32768 // 128 + 1) * 128 * 128 * 2
        assert need <= lay.part_lse - lay.v_wide < need + 256
    ragged = msa.make_shape(batch=3, total_q=700, total_k=1000, max_q=400, max_k=500, hq=8,
                            hkv=2, topk=4, dp=32)
    lay = msa.msa_workspace_layout_of(ragged, msa.MSA_KV_OUTER)
    assert lay.part_lse - lay.v_wide >= 2 * (8 + 3) * 128 * 128 * 2
    lq = msa.msa_workspace_layout_of(m3_shape(), msa.MSA_Q_OUTER)
    assert lq.v_wide == 0 or lq.part_lse - lq.v_wide < 256


def test_partial_memory_ratio_matches_the_pages():
    """bf16 partials of every selected block take topk times the bf16 output."""
    g = json.load(open(GOLDEN))["partial_memory_ratio"]
    s = m3_shape(topk=g["topk"])
    lay = msa.msa_workspace_layout_of(s, msa.MSA_KV_OUTER)
    part_o_bytes = lay.total - lay.part_o               # the partials close the workspace
    out_bytes = 32768 * 64 * 128 * 2
    assert part_o_bytes - out_bytes * g["bf16_partials_over_bf16_output"] in range(0, 256)


def test_query_range_rule():
    """Ranges hold the longest of 1024 (bf16) or 2048 (fp8) .. 512 queries that leaves at least
    128 (sequence, group, range) phases."""
    def q_range(s):
        lay = msa.msa_workspace_layout_of(s, msa.MSA_KV_OUTER)
        return 64 * lay.words_per_bucket, lay.n_ranges
    fp8 = msa.MSA_FP8_E4M3
    assert q_range(m3_shape()) == (1024, 32)                     # 4 groups x 32 ranges
    long = dict(total_q=131072, total_k=131072, max_q=131072, max_k=131072)
    assert q_range(m3_shape(dtype=fp8, **long)) == (2048, 64)
    assert q_range(m3_shape(**long)) == (1024, 128)
    assert q_range(m3_shape(total_q=4096, total_k=4096, max_q=4096, max_k=4096)) == (512, 8)
    assert q_range(m3_shape(dtype=fp8)) == (1024, 32)            # 4 groups x 32 ranges
    # 32 sequences of at most 2048 queries, 2 groups: 1024-query ranges (32 x 2 x 2 = 128)
    many = msa.make_shape(batch=32, total_q=8000, total_k=9000, max_q=2048, max_k=2348, hq=8,
                          hkv=2, topk=5, dp=32, dtype=fp8)
    assert q_range(many) == (1024, 2)
    small = msa.make_shape(batch=1, total_q=1024, total_k=1024, max_q=1024, max_k=1024, hq=32,
                           hkv=2, topk=6, dp=64, dtype=fp8)
    assert q_range(small) == (512, 2)


def test_q_outer_workspace():
    # bf16 per-query lists: splits up to one workgroup per CU of a 256-CU part (the bf16 kernel
    # holds two blocks in LDS); 64 requests x 4 groups already fill it, so the output is
    # written directly
    s = decode_shape()
    lay = msa.msa_workspace_layout_of(s, msa.MSA_Q_OUTER)
    assert lay.slots == 1 and lay.total <= 1024
    few = msa.make_shape(batch=8, total_q=8, total_k=8 * 70000, max_q=1, max_k=131072,
                         hq=64, hkv=4, topk=16, dp=64)
    lay = msa.msa_workspace_layout_of(few, msa.MSA_Q_OUTER)
    assert lay.slots == 8                       # 8 x 4 x 8 = 256 workgroups
    assert lay.part_o - lay.part_lse >= 8 * 4 * lay.slots * 16 * 4
    # fp8 (one block in LDS, two workgroups per CU): about 512 workgroups
    f8 = msa.make_shape(batch=64, total_q=64, total_k=64 * 70000, max_q=1, max_k=131072,
                        hq=64, hkv=4, topk=16, dp=64, dtype=msa.MSA_FP8_E4M3)
    lay = msa.msa_workspace_layout_of(f8, msa.MSA_Q_OUTER)
    assert lay.slots == 2
    assert lay.part_o - lay.part_lse >= 64 * 4 * lay.slots * 16 * 4
    tiles = msa.make_shape(batch=1, total_q=8192, total_k=8192, max_q=8192, max_k=8192, hq=16,
                           hkv=16, topk=16, causal=False, list_q=128)
    lt = msa.msa_workspace_layout_of(tiles, msa.MSA_Q_OUTER)
    assert lt.slots == 1 and lt.total <= 1024  # output written directly, nothing else


# ------------------------------------------------------------------ schedule rule


def test_dispatch_rule():
    assert msa.msa_resolve_mode(m3_shape(), msa.MSA_AUTO) == msa.MSA_KV_OUTER
    assert msa.msa_resolve_mode(m3_shape(dtype=msa.MSA_FP8_E4M3, total_q=131072, max_q=131072,
                                         total_k=131072, max_k=131072),
                                msa.MSA_AUTO) == msa.MSA_KV_OUTER
    assert msa.msa_resolve_mode(decode_shape(), msa.MSA_AUTO) == msa.MSA_Q_OUTER
    tiles = msa.make_shape(batch=1, total_q=8192, total_k=8192, max_q=8192, max_k=8192, hq=16,
                           hkv=16, topk=16, causal=False, list_q=128)
    assert msa.msa_resolve_mode(tiles, msa.MSA_AUTO) == msa.MSA_Q_OUTER
    # explicit modes are honoured
    assert msa.msa_resolve_mode(decode_shape(), msa.MSA_KV_OUTER) == msa.MSA_KV_OUTER
    assert msa.msa_resolve_mode(m3_shape(), msa.MSA_Q_OUTER) == msa.MSA_Q_OUTER


def test_crossover_reproduces_the_pages_figure():
    g = json.load(open(GOLDEN))["crossover"]
    s = msa.make_shape(batch=1, total_q=1024, total_k=1024, max_q=1024, max_k=1024, hq=g["hq"],
                       hkv=g["hkv"], topk=g["topk"], dtype=msa.MSA_FP8_E4M3)
    x = msa.msa_crossover(s, g["hbm_tbps"], g["l2_tbps"])
    assert abs(x / g["nsb_over_n"] - 1) <= g["relative_tolerance"], x


def test_crossover_is_monotone_in_cache_bandwidth():
    s = m3_shape()
    xs = [msa.msa_crossover(s, 8.0, b) for b in (10.0, 16.0, 24.0)]
    assert xs[0] > xs[1] > xs[2]
    s8 = m3_shape(dtype=msa.MSA_FP8_E4M3)
    # fp8 data halves the K/V bytes Q-outer re-reads: the crossover moves down
    assert msa.msa_crossover(s8, 8.0, 16.0) < xs[1]


def test_backward_argument_checks(L):
    """bf16 only; every pointer and the workspace checked before any launch; the workspace
    holds the KV-outer plan plus fp32 dQ partials of every (query-group, block) entry."""
    fake = ctypes.c_void_p(0x1000)
    s = m3_shape()
    need = msa.msa_bwd_workspace_size(s)
    fwd = msa.msa_workspace_size(s, msa.MSA_KV_OUTER)
    lay = msa.msa_workspace_layout_of(s, msa.MSA_KV_OUTER)
    e_max = s.total_q * s.hkv * s.topk
    # plan, bf16 dQ partials, and per chunk of 4096 rows (at most E / 256 + 4 x 256 chunks at
    # G = 16) its column and a 128 KiB dK / dV partial
    chunks = e_max // 256 + 4 * 256
    extra = need - fwd - e_max * (s.hq // s.hkv) * 128 * 2
    assert extra - ((4 * 256 + 1) * 4 + chunks * 4 + chunks * 2 * 128 * 128 * 4) in range(0, 1024)
    assert lay.part_lse + s.total_q * s.hq * 4 <= lay.part_l     # the D rows fit the LSE region

    def bwd(shape, ws=fake, nbytes=need, q=fake, dout=fake, dk=fake, lists=fake):
        return L.msa_sparse_attn_bwd(ctypes.byref(shape), q, fake, fake, fake, fake, dout, 0.1,
                                     lists, fake, fake, ws, nbytes, fake, dk, fake, None)
    assert bwd(m3_shape(dtype=msa.MSA_FP8_E4M3)) == msa.MSA_ERR_DTYPE
    assert bwd(s, q=None) == msa.MSA_ERR_NULL
    assert bwd(s, dout=None) == msa.MSA_ERR_NULL
    assert bwd(s, dk=None) == msa.MSA_ERR_NULL
    assert bwd(s, lists=None) == msa.MSA_ERR_NULL
    assert bwd(s, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE
    assert bwd(s, ws=None) == msa.MSA_ERR_WORKSPACE
    n = ctypes.c_size_t(0)
    assert L.msa_bwd_workspace_size(ctypes.byref(m3_shape(dtype=msa.MSA_FP8_E4M3)),
                                    ctypes.byref(n)) == msa.MSA_ERR_DTYPE


def test_proxy_backward_argument_checks(L):
    """bf16, dp 32 or 64; pointers and workspace checked before any launch."""
    fake = ctypes.c_void_p(0x1000)
    s = m3_shape()
    need = msa.msa_proxy_bwd_workspace_size(s)
    e_max = s.total_q * s.hkv * s.topk
    # at least the plan, the fp32 dq_idx partials and the proxy LSE
    assert need >= msa.msa_workspace_size(s, msa.MSA_KV_OUTER) + e_max * 64 * 4 + s.total_q * 4 * 4

    def pb(shape, ws=fake, nbytes=need, qi=fake, dki=fake):
        return L.msa_proxy_attn_bwd(ctypes.byref(shape), fake, fake, qi, fake, fake, 0.1, 0.125,
                                    fake, fake, fake, ws, nbytes, fake, dki, None, None)
    assert pb(m3_shape(dtype=msa.MSA_FP8_E4M3)) == msa.MSA_ERR_DTYPE
    assert pb(s, qi=None) == msa.MSA_ERR_NULL
    assert pb(s, dki=None) == msa.MSA_ERR_NULL
    assert pb(s, nbytes=need - 1) == msa.MSA_ERR_WORKSPACE
    assert pb(s, ws=None) == msa.MSA_ERR_WORKSPACE


def test_noalloc_rejects_shapes_beyond_its_scratch_without_a_gpu(L):
    """The allocation-free call checks the shape and the scratch size on the host first: a
    shape whose workspace exceeds MSA_NOALLOC_SCRATCH_BYTES returns MSA_ERR_WORKSPACE with the
    byte counts in msa_last_error, before any device call."""
    import ctypes
    big = msa.make_shape(batch=1, total_q=32768, total_k=32768, max_q=32768, max_k=32768,
                         hq=64, hkv=4, topk=16, dp=64)
    st = L.msa_sparse_attn_fwd_noalloc(ctypes.byref(big), None, None, None, None, 0.1, None,
                                       None, None, msa.MSA_KV_OUTER, None, None, None)
    assert st == msa.MSA_ERR_WORKSPACE
    assert b"scratch" in L.msa_last_error()
    st = L.msa_sparse_attn_fwd_noalloc(None, None, None, None, None, 0.1, None, None, None,
                                       msa.MSA_KV_OUTER, None, None, None)
    assert st == msa.MSA_ERR_NULL


def test_probe_argument_checks(L):
    """The bandwidth probe rejects missing buffers and working sets below one pass (4 MiB) or
    not a multiple of 4 KiB, before any launch."""
    import ctypes
    one = ctypes.c_void_p(1)
    assert L.msa_probe_read(None, 4 << 20, 4 << 20, one, None) == msa.MSA_ERR_NULL
    assert L.msa_probe_read(one, 4 << 20, 4 << 20, None, None) == msa.MSA_ERR_NULL
    assert L.msa_probe_read(one, (4 << 20) - 4096, 4 << 20, one, None) == msa.MSA_ERR_SHAPE
    assert L.msa_probe_read(one, (4 << 20) + 100, 8 << 20, one, None) == msa.MSA_ERR_SHAPE
    assert L.msa_probe_read(one, 4 << 20, (4 << 20) - 1, one, None) == msa.MSA_ERR_SHAPE


def test_default_cache_ratio_is_the_measured_one():
    """bw_cache = 0 selects the ratio measured on MI355X (2.32: the model's crossover then
    equals the one timed there, nsb/N = 19.2), and AUTO decides with it."""
    s = m3_shape()
    x_default = msa.msa_crossover(s, 1.0, 0.0)
    assert abs(x_default - msa.msa_crossover(s, 1.0, 2.32)) < 1e-9
    assert abs(x_default - 19.2) < 0.1
    # a list reuse just above / below the crossover picks Q-outer / KV-outer
    def reuse_shape(n_q):
        n = 2048
        return msa.make_shape(batch=n // n_q, total_q=n, total_k=n // n_q * 2048, max_q=n_q,
                              max_k=2048, hq=64, hkv=4, topk=16, causal=False)
    assert msa.msa_resolve_mode(reuse_shape(2), msa.MSA_AUTO) == msa.MSA_Q_OUTER    # 32
    assert msa.msa_resolve_mode(reuse_shape(4), msa.MSA_AUTO) == msa.MSA_KV_OUTER   # 16


def test_index_workspace_covers_every_key_chunk():
    """Short-query calls write one top-16 list (score + id, 8 bytes a slot) per (query, group,
    key chunk): chunks of 8 blocks up to 1024 blocks, 32 beyond."""
    for max_k, per in ((1000, 8), (1024 * 128, 8), (1025 * 128, 32), (300000, 32)):
        s = msa.make_shape(batch=3, total_q=5, total_k=3 * max_k, max_q=2, max_k=max_k, hq=8,
                           hkv=4, topk=16)
        nb = -(-max_k // 128)
        assert msa.msa_index_workspace_size(s) == 3 * 2 * 4 * (-(-nb // per)) * 16 * 8 + 256
