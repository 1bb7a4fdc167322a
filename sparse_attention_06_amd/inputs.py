"""Seeded synthetic inputs for the DeepSeek Sparse Attention (DSA) hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scores, no selection, no attention). Both the float64
CPU oracle (through the tests and the bench's CPU leg) and the HIP path are fed
from here, so neither side ever generates inputs for the other.

Recipe (the workloads of "DeepSeek3.2: Onboard sparse attention", section
"What this PR does", item 2, for the index shapes; "Integrate DeepSeek Sparse
Attention with Tokamax Flash Attention", section "Description", for the 2B
batch-12 / seq-4096 run):

* every tensor has its own generator, seeded from ``(seed, tensor_id)``;
* q, k, v, q_idx, k_idx are N(0, 1) multiplied by ``last_dim ** -0.5`` when
  ``scaled`` is set (all bf16 configurations), unscaled otherwise;
* w (per-token, per-index-head weight) is N(0, 1/Hi), i.e. std ``Hi ** -0.5``;
* dO is N(0, 1), unscaled;
* samples are drawn in float32 and rounded to the storage dtype with
  round-to-nearest-even (torch's float32 -> bfloat16 conversion);
* packed-document segment IDs: per batch row, document lengths are drawn
  uniformly from [lo, hi] (inclusive) until the next one would reach or pass
  S; the tail then forms the last document. IDs count up from 1.

Tensors are produced with torch on the requested device (CPU for the small
oracle cases, the GPU for full-size cases, where drawing hundreds of millions
of samples on the host would take minutes). The values differ between devices
but the distributions and shapes do not.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# tensor ids of the per-tensor generator streams
_TID = {"q": 0, "k": 1, "v": 2, "q_idx": 3, "k_idx": 4, "w": 5, "dout": 6,
        "seg": 7, "sets": 8}


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shapes, dtype and the options of its input recipe."""
    name: str
    B: int
    S: int
    Hi: int          # index heads
    Di: int          # index head dim
    K: int           # top-k
    H: int           # attention heads
    Dqk: int         # query/key head dim
    Dv: int          # value head dim
    dtype: str       # "bf16" or "fp32" (storage and compute-input type)
    scaled: bool     # scale q,k,v,q_idx,k_idx by last_dim ** -0.5
    segments: Optional[tuple] = None   # (lo, hi) document-length range, or None
    backward: bool = False
    score_dtype: str = "fp32"
    seed: int = 0
    ratio: int = 1   # keys are compressed blocks of `ratio` tokens (1: token-level DSA)

    @property
    def Sk(self) -> int:
        """Keys per batch row: S tokens, or S // ratio compressed entries."""
        return self.S // self.ratio

    @property
    def softmax_scale(self) -> float:
        return float(self.Dqk) ** -0.5

    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads. c1 is the tiny fp32 unit-test shape (seq 128), c2 the
# 2B-model training shape (batch 12, seq 4096), c3 the 671B head count at 32K,
# c4 packed documents, c5 the 128K long-context case with bf16 scores.
CONFIGS = {
    "c1": Config("c1_tiny_fp32", 1, 128, 4, 32, 16, 2, 64, 64, "fp32", False),
    "c2": Config("c2_2b_b12_s4k", 12, 4096, 64, 128, 2048, 16, 192, 128, "bf16", True,
                 backward=True),
    "c3": Config("c3_671b_heads_s32k", 1, 32768, 64, 128, 2048, 128, 192, 128, "bf16", True),
    "c4": Config("c4_packed_b4_s8k", 4, 8192, 64, 128, 2048, 32, 192, 128, "bf16", True,
                 segments=(64, 4096), backward=True),
    "c5": Config("c5_long_s128k", 1, 131072, 64, 128, 2048, 128, 192, 128, "bf16", True,
                 score_dtype="bf16"),
}

# Compressed sparse attention (DeepSeek-V4 CSA, compression ratio 4) on the 2B
# shape: 1024 compressed entries per row of 4096 tokens; top-k scaled by the
# ratio (2048 / 4). Forward by default (`.replace(backward=True)` adds dO).
# Not one of the five metric workloads.
CSA_CONFIGS = {
    "csa": Config("csa_r4_b12_s4k", 12, 4096, 64, 128, 512, 16, 192, 128, "bf16", True, ratio=4),
}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + _TID[name] * 7919 + 17)
    return g


def normal(shape, sigma: float, seed: int, name: str, dtype, device="cpu") -> torch.Tensor:
    """N(0, sigma^2) drawn in float32 on ``device``, then rounded to ``dtype``."""
    g = _gen(seed, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def segment_ids(B: int, S: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Packed-document segment IDs [B, S] int32 (IDs 1, 2, ... per row)."""
    seg = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        rng = np.random.default_rng(np.random.SeedSequence([seed, _TID["seg"], b]))
        start, doc = 0, 1
        while start < S:
            n = int(rng.integers(lo, hi + 1))
            end = start + n
            if end >= S:
                end = S
            seg[b, start:end] = doc
            start, doc = end, doc + 1
    return seg


def make(cfg: Config, device="cpu", with_dout: Optional[bool] = None) -> dict:
    """All inputs of one configuration as torch tensors on ``device``."""
    dt = cfg.torch_dtype()
    B, S = cfg.B, cfg.S

    def sig(d):
        return float(d) ** -0.5 if cfg.scaled else 1.0

    Sk = cfg.Sk  # key-side rows: tokens, or compressed entries
    out = {
        "q": normal((B, S, cfg.H, cfg.Dqk), sig(cfg.Dqk), cfg.seed, "q", dt, device),
        "k": normal((B, Sk, cfg.H, cfg.Dqk), sig(cfg.Dqk), cfg.seed, "k", dt, device),
        "v": normal((B, Sk, cfg.H, cfg.Dv), sig(cfg.Dv), cfg.seed, "v", dt, device),
        "q_idx": normal((B, S, cfg.Hi, cfg.Di), sig(cfg.Di), cfg.seed, "q_idx", dt, device),
        "k_idx": normal((B, Sk, cfg.Di), sig(cfg.Di), cfg.seed, "k_idx", dt, device),
        "w": normal((B, S, cfg.Hi), float(cfg.Hi) ** -0.5, cfg.seed, "w", dt, device),
    }
    if with_dout is None:
        with_dout = cfg.backward
    if with_dout:
        out["dout"] = normal((B, S, cfg.H, cfg.Dv), 1.0, cfg.seed, "dout", dt, device)
    if cfg.segments is not None:
        seg = segment_ids(B, S, cfg.segments[0], cfg.segments[1], cfg.seed)
        out["seg"] = torch.from_numpy(seg).to(device)
    else:
        out["seg"] = None
    return out


def make_index_inputs(cfg: Config, device="cpu") -> dict:
    """Only the indexer's inputs (q_idx, k_idx, w, seg) of a configuration:
    the same tensors, drawn from the same streams, as ``make`` returns."""
    dt = cfg.torch_dtype()
    B, S = cfg.B, cfg.S
    sig = float(cfg.Di) ** -0.5 if cfg.scaled else 1.0
    out = {
        "q_idx": normal((B, S, cfg.Hi, cfg.Di), sig, cfg.seed, "q_idx", dt, device),
        "k_idx": normal((B, S, cfg.Di), sig, cfg.seed, "k_idx", dt, device),
        "w": normal((B, S, cfg.Hi), float(cfg.Hi) ** -0.5, cfg.seed, "w", dt, device),
    }
    if cfg.segments is not None:
        seg = segment_ids(B, S, cfg.segments[0], cfg.segments[1], cfg.seed)
        out["seg"] = torch.from_numpy(seg).to(device)
    else:
        out["seg"] = None
    return out


def random_index_sets(B: int, S: int, K: int, seg: Optional[np.ndarray], seed: int,
                      rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Uniformly random key sets, one per query row, as a sparsity pattern.

    Row t draws min(K, m) distinct keys without replacement from the m keys
    at or before t that carry t's segment ID (all keys at or before t when
    ``seg`` is None), sorted ascending and padded with -1 to K entries.
    Returns int32 [B, len(rows), K]. This is a pattern generator for the
    attention kernels' inputs, not the method's selection rule.
    """
    if rows is None:
        rows = np.arange(S)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, K), -1, dtype=np.int32)
    for b in range(B):
        # one generator per row, so that a row subset matches the full draw
        for i, t in enumerate(rows):
            rrng = np.random.default_rng(np.random.SeedSequence([seed, _TID["sets"], b, int(t)]))
            if seg is None:
                cand = np.arange(int(t) + 1)
            else:
                cand = np.nonzero(seg[b, : int(t) + 1] == seg[b, int(t)])[0]
            n = min(K, cand.size)
            pick = np.sort(rrng.choice(cand, size=n, replace=False)) if n < cand.size else cand
            out[b, i, :n] = pick
    return out
