"""ctypes binding of libmsa (include/msa.h): argument marshalling only.

Every function has the name and argument order of its C counterpart; tensors are passed as
device pointers and the stream defaults to torch's current HIP stream. Nothing here computes
any part of the method: a missing libmsa.so raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa.so")

MSA_OK, MSA_ERR_NULL, MSA_ERR_SHAPE, MSA_ERR_DTYPE, MSA_ERR_WORKSPACE, MSA_ERR_MODE, \
    MSA_ERR_LAUNCH = range(7)
MSA_BF16, MSA_FP8_E4M3 = 0, 1
MSA_AUTO, MSA_KV_OUTER, MSA_Q_OUTER = 0, 1, 2

SYMBOLS = ("msa_workspace_size", "msa_workspace_layout_of", "msa_index_workspace_size",
           "msa_resolve_mode", "msa_crossover", "msa_status_string", "msa_last_error",
           "msa_index_topk", "msa_index_topk_fp8", "msa_index_topk_mxfp4", "msa_sparse_attn_fwd", "msa_plan",
           "msa_attn_main", "msa_combine", "msa_select_workspace_size", "msa_select_tiles",
           "msa_bwd_workspace_size", "msa_sparse_attn_bwd", "msa_proxy_bwd_workspace_size",
           "msa_proxy_attn_bwd", "msa_train_bwd_workspace_size", "msa_train_bwd",
           "msa_sparse_attn_fwd_noalloc", "msa_probe_read")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "total_q", "total_k", "max_q", "max_k", "hq", "hkv", "d", "dp", "block",
        "topk", "causal", "dtype", "list_q")]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "counters", "masks", "offsets", "scan_sums", "entry_q", "entry_bucket", "cmap",
        "part_lse", "part_l", "part_o", "v_wide", "total")] + [(n, ctypes.c_int32) for n in (
            "slots", "n_words", "w_max", "nb_max", "words_per_bucket", "n_ranges")]


class MSAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_sparse_gqa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        sp = ctypes.POINTER(Shape)
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_status_string.argtypes = [i32]
        L.msa_last_error.restype = ctypes.c_char_p
        L.msa_last_error.argtypes = []
        for name, args in {
            "msa_workspace_size": [sp, i32, ctypes.POINTER(sz)],
            "msa_workspace_layout_of": [sp, i32, ctypes.POINTER(WorkspaceLayout)],
            "msa_index_workspace_size": [sp, ctypes.POINTER(sz)],
            "msa_resolve_mode": [sp, i32, ctypes.POINTER(i32)],
            "msa_crossover": [sp, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)],
            "msa_index_topk": [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_index_topk_fp8": [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_index_topk_mxfp4": [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_select_workspace_size": [sp, i32, ctypes.POINTER(sz)],
            "msa_select_tiles": [sp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
            "msa_sparse_attn_fwd": [sp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, i32, vp, sz,
                                    vp, vp, vp],
            "msa_plan": [sp, vp, vp, vp, vp, sz, vp],
            "msa_attn_main": [sp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp],
            "msa_combine": [sp, i32, vp, sz, vp, vp, vp],
            "msa_probe_read": [vp, sz, sz, vp, vp],
            "msa_sparse_attn_fwd_noalloc": [sp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, i32,
                                            vp, vp, vp],
            "msa_bwd_workspace_size": [sp, ctypes.POINTER(sz)],
            "msa_proxy_bwd_workspace_size": [sp, ctypes.POINTER(sz)],
            "msa_train_bwd_workspace_size": [sp, ctypes.POINTER(sz)],
            "msa_train_bwd": [sp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, ctypes.c_float,
                              vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp],
            "msa_proxy_attn_bwd": [sp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp,
                                   vp, vp, vp, sz, vp, vp, vp, vp],
            "msa_sparse_attn_bwd": [sp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                    sz, vp, vp, vp, vp],
        }.items():
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = args
        _lib = L
    return _lib


def _check(st: int, where: str) -> None:
    if st != MSA_OK:
        L = lib()
        detail = L.msa_status_string(st).decode()
        if st == MSA_ERR_LAUNCH or (st == MSA_ERR_WORKSPACE and where.endswith("_noalloc")):
            detail += ": " + L.msa_last_error().decode()
        raise MSAError(st, where, detail)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t                      # already a raw pointer (int) or None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_shape(*, batch, total_q, total_k, max_q, max_k, hq, hkv, topk, d=128, dp=64,
               block=128, causal=True, dtype=MSA_BF16, list_q=1) -> Shape:
    return Shape(batch, total_q, total_k, max_q, max_k, hq, hkv, d, dp, block, topk,
                 int(bool(causal)), dtype, list_q)


# ------------------------------------------------------------------ host-only queries

def msa_workspace_size(shape: Shape, mode: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_workspace_size(ctypes.byref(shape), mode, ctypes.byref(n)), "msa_workspace_size")
    return n.value


def msa_workspace_layout_of(shape: Shape, mode: int) -> WorkspaceLayout:
    out = WorkspaceLayout()
    _check(lib().msa_workspace_layout_of(ctypes.byref(shape), mode, ctypes.byref(out)),
           "msa_workspace_layout_of")
    return out


def msa_index_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_index_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "msa_index_workspace_size")
    return n.value


def msa_resolve_mode(shape: Shape, mode: int) -> int:
    out = ctypes.c_int(0)
    _check(lib().msa_resolve_mode(ctypes.byref(shape), mode, ctypes.byref(out)), "msa_resolve_mode")
    return out.value


def msa_crossover(shape: Shape, bw_hbm: float, bw_cache: float) -> float:
    out = ctypes.c_double(0)
    _check(lib().msa_crossover(ctypes.byref(shape), bw_hbm, bw_cache, ctypes.byref(out)),
           "msa_crossover")
    return out.value


# ------------------------------------------------------------------ device calls

def msa_index_topk(shape, q_idx, k_idx, cu_q, cu_k, topk_idx, topk_score=None, workspace=None,
                   stream=None) -> None:
    _check(lib().msa_index_topk(ctypes.byref(shape), _p(q_idx), _p(k_idx), _p(cu_q), _p(cu_k),
                                _p(topk_idx), _p(topk_score), _p(workspace), _nbytes(workspace),
                                _stream(stream)), "msa_index_topk")


def msa_index_topk_fp8(shape, q_idx, k_idx, descale_idx, cu_q, cu_k, topk_idx, topk_score=None,
                       workspace=None, stream=None) -> None:
    _check(lib().msa_index_topk_fp8(ctypes.byref(shape), _p(q_idx), _p(k_idx), _p(descale_idx),
                                    _p(cu_q), _p(cu_k), _p(topk_idx), _p(topk_score),
                                    _p(workspace), _nbytes(workspace), _stream(stream)),
           "msa_index_topk_fp8")


def msa_index_topk_mxfp4(shape, q_idx, q_scale, k_idx, k_scale, cu_q, cu_k, topk_idx,
                         topk_score=None, workspace=None, stream=None) -> None:
    _check(lib().msa_index_topk_mxfp4(ctypes.byref(shape), _p(q_idx), _p(q_scale), _p(k_idx),
                                      _p(k_scale), _p(cu_q), _p(cu_k), _p(topk_idx),
                                      _p(topk_score), _p(workspace), _nbytes(workspace),
                                      _stream(stream)),
           "msa_index_topk_mxfp4")


def msa_select_workspace_size(shape, reps) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_select_workspace_size(ctypes.byref(shape), int(reps), ctypes.byref(n)),
           "msa_select_workspace_size")
    return n.value


def msa_select_tiles(shape, reps, q, k, cu_q, cu_k, lists, scores=None, workspace=None,
                     stream=None) -> None:
    _check(lib().msa_select_tiles(ctypes.byref(shape), int(reps), _p(q), _p(k), _p(cu_q),
                                  _p(cu_k), _p(lists), _p(scores), _p(workspace),
                                  _nbytes(workspace), _stream(stream)), "msa_select_tiles")


def msa_sparse_attn_fwd(shape, q, k, v, descale_qkv, softmax_scale, topk_idx, cu_q, cu_k, mode,
                        workspace, o, lse, stream=None) -> None:
    _check(lib().msa_sparse_attn_fwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(descale_qkv),
                                     float(softmax_scale), _p(topk_idx), _p(cu_q), _p(cu_k), mode,
                                     _p(workspace), _nbytes(workspace), _p(o), _p(lse),
                                     _stream(stream)), "msa_sparse_attn_fwd")


def msa_plan(shape, topk_idx, cu_q, cu_k, workspace, stream=None) -> None:
    _check(lib().msa_plan(ctypes.byref(shape), _p(topk_idx), _p(cu_q), _p(cu_k), _p(workspace),
                          _nbytes(workspace), _stream(stream)), "msa_plan")


def msa_attn_main(shape, q, k, v, descale_qkv, softmax_scale, cu_q, cu_k, workspace,
                  stream=None) -> None:
    _check(lib().msa_attn_main(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(descale_qkv),
                               float(softmax_scale), _p(cu_q), _p(cu_k), _p(workspace),
                               _nbytes(workspace), _stream(stream)), "msa_attn_main")


def msa_combine(shape, mode, workspace, o, lse, stream=None) -> None:
    _check(lib().msa_combine(ctypes.byref(shape), mode, _p(workspace), _nbytes(workspace), _p(o),
                             _p(lse), _stream(stream)), "msa_combine")


def msa_sparse_attn_fwd_noalloc(shape, q, k, v, descale_qkv, softmax_scale, topk_idx, cu_q, cu_k,
                                mode, o, lse, stream=None) -> None:
    _check(lib().msa_sparse_attn_fwd_noalloc(ctypes.byref(shape), _p(q), _p(k), _p(v),
                                             _p(descale_qkv), float(softmax_scale), _p(topk_idx),
                                             _p(cu_q), _p(cu_k), mode, _p(o), _p(lse),
                                             _stream(stream)), "msa_sparse_attn_fwd_noalloc")


def msa_probe_read(buf, working_set_bytes, total_bytes, sink, stream=None) -> None:
    _check(lib().msa_probe_read(_p(buf), int(working_set_bytes), int(total_bytes), _p(sink),
                                _stream(stream)), "msa_probe_read")


def msa_bwd_workspace_size(shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "msa_bwd_workspace_size")
    return n.value


def msa_sparse_attn_bwd(shape, q, k, v, o, lse, dout, softmax_scale, topk_idx, cu_q, cu_k,
                        workspace, dq, dk, dv, stream=None) -> None:
    _check(lib().msa_sparse_attn_bwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(o), _p(lse),
                                     _p(dout), float(softmax_scale), _p(topk_idx), _p(cu_q),
                                     _p(cu_k), _p(workspace), _nbytes(workspace), _p(dq), _p(dk),
                                     _p(dv), _stream(stream)), "msa_sparse_attn_bwd")


def msa_proxy_bwd_workspace_size(shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_proxy_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "msa_proxy_bwd_workspace_size")
    return n.value


def msa_proxy_attn_bwd(shape, q, k, q_idx, k_idx, lse, softmax_scale, proxy_scale, topk_idx,
                       cu_q, cu_k, workspace, dq_idx, dk_idx, lse_proxy=None, stream=None) -> None:
    _check(lib().msa_proxy_attn_bwd(ctypes.byref(shape), _p(q), _p(k), _p(q_idx), _p(k_idx),
                                    _p(lse), float(softmax_scale), float(proxy_scale),
                                    _p(topk_idx), _p(cu_q), _p(cu_k), _p(workspace),
                                    _nbytes(workspace), _p(dq_idx), _p(dk_idx), _p(lse_proxy),
                                    _stream(stream)), "msa_proxy_attn_bwd")


def msa_train_bwd_workspace_size(shape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_train_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "msa_train_bwd_workspace_size")
    return n.value


def msa_train_bwd(shape, q, k, v, o, lse, dout, softmax_scale, q_idx, k_idx, proxy_scale,
                  topk_idx, cu_q, cu_k, workspace, dq, dk, dv, dq_idx, dk_idx, lse_proxy=None,
                  stream=None) -> None:
    _check(lib().msa_train_bwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(o), _p(lse),
                               _p(dout), float(softmax_scale), _p(q_idx), _p(k_idx),
                               float(proxy_scale), _p(topk_idx), _p(cu_q), _p(cu_k),
                               _p(workspace), _nbytes(workspace), _p(dq), _p(dk), _p(dv),
                               _p(dq_idx), _p(dk_idx), _p(lse_proxy), _stream(stream)),
           "msa_train_bwd")
