"""The whole MSA layer call on torch-allocated device buffers.

index branch (msa_index_topk) -> main branch (msa_sparse_attn_fwd) -> combine (msa_combine),
all enqueued on one stream with no host synchronisation. Buffers are allocated with torch
and cached per shape, so repeated calls of one shape allocate nothing.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

from . import msa


@dataclass
class Buffers:
    topk_idx: Optional[torch.Tensor] = None
    topk_score: Optional[torch.Tensor] = None
    index_ws: Optional[torch.Tensor] = None
    ws: Optional[torch.Tensor] = None
    o: Optional[torch.Tensor] = None
    lse: Optional[torch.Tensor] = None


@dataclass
class MSALayer:
    """Block-sparse GQA attention layer for one fixed shape (see include/msa.h)."""
    shape: msa.Shape
    mode: int = msa.MSA_AUTO
    softmax_scale: float = 128 ** -0.5
    want_scores: bool = False
    bufs: Buffers = field(default_factory=Buffers)

    def __post_init__(self):
        self.chosen = msa.msa_resolve_mode(self.shape, self.mode)

    def _alloc(self, device) -> Buffers:
        s, b = self.shape, self.bufs
        if b.o is None:
            n_lists = s.total_q
            b.topk_idx = torch.empty((n_lists, s.hkv, s.topk), dtype=torch.int32, device=device)
            if self.want_scores:
                b.topk_score = torch.empty((n_lists, s.hkv, s.topk), dtype=torch.float32,
                                           device=device)
            nidx = msa.msa_index_workspace_size(s) if s.list_q == 1 else 0
            b.index_ws = torch.empty(max(nidx, 256), dtype=torch.uint8, device=device)
            b.ws = torch.empty(msa.msa_workspace_size(s, self.chosen), dtype=torch.uint8,
                               device=device)
            b.o = torch.empty((s.total_q, s.hq, s.d), dtype=torch.bfloat16, device=device)
            b.lse = torch.empty((s.total_q, s.hq), dtype=torch.float32, device=device)
        return b

    def index(self, q_idx, k_idx, cu_q, cu_k, stream=None) -> torch.Tensor:
        b = self._alloc(cu_q.device)
        msa.msa_index_topk(self.shape, q_idx, k_idx, cu_q, cu_k, b.topk_idx, b.topk_score,
                           b.index_ws, stream)
        return b.topk_idx

    def attend(self, q, k, v, lists, cu_q, cu_k, descale=None, stream=None):
        b = self._alloc(cu_q.device)
        msa.msa_sparse_attn_fwd(self.shape, q, k, v, descale, self.softmax_scale, lists, cu_q,
                                cu_k, self.chosen, b.ws, b.o, b.lse, stream)
        msa.msa_combine(self.shape, self.chosen, b.ws, b.o, b.lse, stream)
        return b.o, b.lse

    def forward(self, q, k, v, q_idx, k_idx, cu_q, cu_k, descale=None, lists=None, stream=None):
        """Index branch (unless per-tile ``lists`` are given), then attention and combine."""
        if lists is None:
            lists = self.index(q_idx, k_idx, cu_q, cu_k, stream)
        return self.attend(q, k, v, lists, cu_q, cu_k, descale, stream)
