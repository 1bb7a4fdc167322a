"""The DSA hot path as one object: device buffers plus the five C-ABI calls.

Buffers come from torch (device memory and the current stream). Every
computation is a libdsa call through ``sparse_attention_06_amd.dsa``.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import dsa


class DSAPath:
    """Buffers and calls for one shape: indexer -> top-k -> attention fwd [-> bwd].

    ``score_rows`` bounds the score buffer to a slab of rows (a multiple of
    128). The indexer and top-k then run slab by slab, as the C ABI allows.
    """

    def __init__(self, B, S, Hi, Di, K, H, Dqk, Dv, dtype=torch.bfloat16, score_dtype=torch.float32,
                 device="cuda", backward=False, score_rows: Optional[int] = None):
        self.B, self.S, self.Hi, self.Di, self.K = B, S, Hi, Di, K
        self.H, self.Dqk, self.Dv = H, Dqk, Dv
        self.dtype, self.score_dtype, self.device = dtype, score_dtype, device
        rows = S if score_rows is None else min(S, score_rows)
        if rows != S and rows % dsa.TILE_Q:
            raise ValueError("score_rows must be a multiple of 128")
        self.slab = rows
        self.scores = torch.empty((B, rows, S), dtype=score_dtype, device=device)
        self.idx = torch.empty((B, S, K), dtype=torch.int32, device=device)
        self.mask = torch.empty(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=device)
        self.o = torch.empty((B, S, H, Dv), dtype=dtype, device=device)
        self.lse = torch.empty((B, H, S), dtype=torch.float32, device=device)
        if backward:
            self.dq = torch.empty((B, S, H, Dqk), dtype=dtype, device=device)
            self.dk = torch.empty((B, S, H, Dqk), dtype=dtype, device=device)
            self.dv = torch.empty((B, S, H, Dv), dtype=dtype, device=device)
            nbytes = dsa.dsa_bwd_workspace_bytes(B, S, H, Dqk, Dv, dtype)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def select(self, q_idx, k_idx, w, seg=None):
        """Indexer scores and top-k for every row (slab by slab)."""
        for row0 in range(0, self.S, self.slab):
            n = min(self.slab, self.S - row0)
            sc = self.scores if n == self.slab else \
                self.scores.view(-1)[: self.B * n * self.S].view(self.B, n, self.S)  # [B, nrows, S]
            dsa.dsa_index_scores(q_idx, k_idx, w, seg, row0, n, sc)
            dsa.dsa_topk(sc, seg, self.B, self.S, self.K, row0, n, self.idx, self.mask)

    def select_fp8(self, q8, q_scale, k8, k_scale, w, seg=None):
        """select() on fp8 (E4M3) index queries and keys with their row scales
        (see dsa_quant_fp8_rows / dsa_index_scores_fp8)."""
        for row0 in range(0, self.S, self.slab):
            n = min(self.slab, self.S - row0)
            sc = self.scores if n == self.slab else \
                self.scores.view(-1)[: self.B * n * self.S].view(self.B, n, self.S)
            dsa.dsa_index_scores_fp8(q8, q_scale, k8, k_scale, w, seg, row0, n, sc)
            dsa.dsa_topk(sc, seg, self.B, self.S, self.K, row0, n, self.idx, self.mask)

    def build_mask(self, idx, seg=None):
        dsa.dsa_build_mask(idx, seg, self.mask)

    def forward(self, q, k, v, scale):
        dsa.dsa_sparse_attn_fwd(q, k, v, self.mask, scale, self.o, self.lse)

    def backward(self, q, k, v, dout, scale):
        dsa.dsa_sparse_attn_bwd(q, k, v, self.o, dout, self.lse, self.mask, scale, self.dq, self.dk,
                                self.dv, self.ws)

    def indexer_loss(self, x: dict, scale: float, inplace: bool = True):
        """The indexer's KL auxiliary loss after forward(): teacher, student
        KL and the gradients of q_idx, k_idx and w. With float32 scores and
        ``inplace``, the score gradient overwrites the scores buffer."""
        B, S, K = self.B, self.S, self.K
        dev = self.device
        if not hasattr(self, "teacher"):
            self.teacher = torch.empty((B, S, K), dtype=torch.float32, device=dev)
            self.row_kl = torch.empty((B, S), dtype=torch.float32, device=dev)
            self.loss = torch.empty(2, dtype=torch.float32, device=dev)
            self.dq_idx = torch.empty(x["q_idx"].shape, dtype=x["q_idx"].dtype, device=dev)
            self.dk_idx = torch.empty(x["k_idx"].shape, dtype=x["k_idx"].dtype, device=dev)
            self.dw = torch.empty(x["w"].shape, dtype=x["w"].dtype, device=dev)
        if self.slab != S:
            raise ValueError("the indexer loss needs the scores of every row (no slabs)")
        if inplace and self.scores.dtype == torch.float32:
            self.dscores = self.scores
        elif getattr(self, "dscores", None) is None or self.dscores is self.scores:
            self.dscores = torch.empty((B, S, S), dtype=torch.float32, device=dev)
        dsa.dsa_indexer_teacher(x["q"], x["k"], self.lse, self.mask, K, scale, self.teacher)
        dsa.dsa_indexer_kl(self.scores, self.idx, self.teacher, self.mask, self.row_kl, self.loss, self.dscores)
        dsa.dsa_indexer_bwd(x["q_idx"], x["k_idx"], x["w"], self.dscores, self.mask, self.dq_idx, self.dk_idx,
                            self.dw)

    def step(self, x: dict, scale: float, backward: bool = False):
        self.select(x["q_idx"], x["k_idx"], x["w"], x.get("seg"))
        self.forward(x["q"], x["k"], x["v"], scale)
        if backward:
            self.backward(x["q"], x["k"], x["v"], x["dout"], scale)
