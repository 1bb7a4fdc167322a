"""ctypes binding of libdsa.so (declared in include/dsa.h).

Argument marshalling only. Each function passes tensor data pointers, sizes
and torch's current HIP stream to the C entry point of the same name, and
raises DSAError on a non-OK status. Every step of the computation runs in the
library's HIP kernels, so a missing library is an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_BF16, DSA_FP32 = 0, 1
TILE_Q, TILE_K = 128, 64
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
          4: "DSA_ERR_HIP"}

EXPORTS = ("dsa_index_scores", "dsa_index_scores_fp8", "dsa_quant_fp8_rows", "dsa_indexer_rope", "dsa_topk", "dsa_build_mask", "dsa_sparse_attn_fwd",
           "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_noalloc", "dsa_sparse_attn_bwd_prep", "dsa_sparse_attn_bwd_dq", "dsa_sparse_attn_bwd_dkdv", "dsa_mask_bytes", "dsa_bwd_workspace_bytes", "dsa_bwd_workspace_min_bytes",
           "dsa_indexer_teacher", "dsa_indexer_kl", "dsa_indexer_bwd",
           "dsa_csa_mask_bytes", "dsa_csa_index_scores", "dsa_csa_topk", "dsa_csa_build_mask", "dsa_csa_sparse_attn_fwd",
           "dsa_csa_sparse_attn_bwd", "dsa_csa_bwd_workspace_bytes",
           "dsa_status_string", "dsa_last_error", "dsa_version")


class DSAError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {detail}")
        self.code = code


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so once. Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_06_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.dsa_index_scores.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, i32, i64, vp]
        L.dsa_index_scores_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, i64, vp]
        L.dsa_quant_fp8_rows.argtypes = [vp, i32, i64, i32, vp, vp, vp]
        L.dsa_indexer_rope.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp]
        L.dsa_topk.argtypes = [vp, i32, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp]
        L.dsa_build_mask.argtypes = [vp, vp, i32, i32, i32, vp, vp]
        L.dsa_sparse_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
        L.dsa_sparse_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                          vp, vp, vp, vp, sz, vp]
        L.dsa_sparse_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                                  i32, vp, vp, vp, vp]
        L.dsa_sparse_attn_bwd_prep.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        L.dsa_indexer_teacher.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
        L.dsa_indexer_kl.argtypes = [vp, i32, i64, vp, vp, vp, i32, i32, i32, vp, vp, vp, i64, vp]
        L.dsa_indexer_bwd.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.dsa_sparse_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                               vp, vp, vp, sz, vp]
        L.dsa_sparse_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                             vp, vp, sz, vp]
        for f in ("dsa_index_scores", "dsa_index_scores_fp8", "dsa_quant_fp8_rows", "dsa_indexer_rope", "dsa_topk", "dsa_build_mask", "dsa_sparse_attn_fwd",
                  "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_noalloc", "dsa_sparse_attn_bwd_prep",
                  "dsa_sparse_attn_bwd_dq",
                  "dsa_sparse_attn_bwd_dkdv", "dsa_indexer_teacher", "dsa_indexer_kl", "dsa_indexer_bwd"):
            getattr(L, f).restype = ctypes.c_int
        L.dsa_csa_index_scores.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, i32, i64,
                                           vp]
        L.dsa_csa_topk.argtypes = [vp, i32, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
        L.dsa_csa_build_mask.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
        L.dsa_csa_sparse_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp,
                                              vp]
        L.dsa_csa_sparse_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                              i32, vp, vp, vp, vp, sz, vp]
        for f in ("dsa_csa_index_scores", "dsa_csa_topk", "dsa_csa_build_mask", "dsa_csa_sparse_attn_fwd",
                  "dsa_csa_sparse_attn_bwd"):
            getattr(L, f).restype = i32
        L.dsa_csa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
        L.dsa_csa_bwd_workspace_bytes.restype = sz
        L.dsa_csa_mask_bytes.argtypes = [i32, i32, i32]
        L.dsa_csa_mask_bytes.restype = sz
        L.dsa_mask_bytes.argtypes = [i32, i32]
        L.dsa_mask_bytes.restype = sz
        L.dsa_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.dsa_bwd_workspace_bytes.restype = sz
        L.dsa_bwd_workspace_min_bytes.argtypes = [i32, i32, i32]
        L.dsa_bwd_workspace_min_bytes.restype = sz
        L.dsa_status_string.argtypes = [i32]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_version.argtypes = []
        L.dsa_version.restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise DSAError(fn, code, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdsa must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t) -> int:
    """DSA dtype code of a tensor or a torch dtype."""
    d = t if isinstance(t, torch.dtype) else t.dtype
    if d == torch.bfloat16:
        return DSA_BF16
    if d == torch.float32:
        return DSA_FP32
    raise ValueError(f"unsupported dtype {d}")


# ------------------------------------------------------------------ sizes
def dsa_mask_bytes(B: int, S: int) -> int:
    return int(lib().dsa_mask_bytes(B, S))


def dsa_bwd_workspace_bytes(B: int, S: int, H: int, Dqk: int, Dv: int, dtype=torch.bfloat16) -> int:
    return int(lib().dsa_bwd_workspace_bytes(B, S, H, Dqk, Dv, _dt(dtype)))


def dsa_bwd_workspace_min_bytes(B: int, S: int, H: int) -> int:
    return int(lib().dsa_bwd_workspace_min_bytes(B, S, H))


def dsa_csa_mask_bytes(B: int, S: int, Sk: int) -> int:
    return int(lib().dsa_csa_mask_bytes(B, S, Sk))


def dsa_csa_bwd_workspace_bytes(B: int, S: int, Sk: int, ratio: int, H: int, Dqk: int, Dv: int,
                                dtype=torch.bfloat16) -> int:
    return int(lib().dsa_csa_bwd_workspace_bytes(B, S, Sk, ratio, H, Dqk, Dv, _dt(dtype)))


def mask_views(mask: torch.Tensor, B: int, S: int, Sk: Optional[int] = None):
    """(sel_bits int64 [B,S,W], tile_cls uint8 [B,NQ,NK]) views of a mask buffer
    (keys: S tokens, or Sk compressed entries)."""
    Sk = S if Sk is None else Sk
    W = (Sk + 63) // 64
    nq, nk = (S + TILE_Q - 1) // TILE_Q, (Sk + TILE_K - 1) // TILE_K
    nb = B * S * W * 8
    bits = mask[:nb].view(torch.int64).view(B, S, W)
    cls = mask[nb:nb + B * nq * nk].view(B, nq, nk)
    return bits, cls


# ------------------------------------------------------------------ calls
def dsa_index_scores(q_idx, k_idx, w, seg, row0: int, nrows: int, scores, stream=None) -> None:
    B, S, Hi, Di = q_idx.shape
    ld = scores.shape[-1]
    _check("dsa_index_scores", lib().dsa_index_scores(
        _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(seg), B, S, Hi, Di, _dt(q_idx), row0, nrows,
        _ptr(scores), _dt(scores), ld, _stream(stream)))


def dsa_quant_fp8_rows(x, codes, scale, stream=None) -> None:
    """Quantize the last axis of x (bf16 or fp32) to E4M3 codes (uint8, same
    shape) with one float32 scale per row (x.shape[:-1])."""
    D = x.shape[-1]
    nrows = x.numel() // D
    _check("dsa_quant_fp8_rows", lib().dsa_quant_fp8_rows(
        _ptr(x), _dt(x), nrows, D, _ptr(codes), _ptr(scale), _stream(stream)))


def dsa_indexer_rope(x, rope_dim: int, cos_t, sin_t, pos=None, out=None, stream=None) -> None:
    """Partial concatenated-layout RoPE of x [B,S,nh,D] or [B,S,D] (bf16) into
    out (default: in place). cos_t, sin_t [P, rope_dim/2] float32."""
    B, S = x.shape[:2]
    nh = x.shape[2] if x.dim() == 4 else 1
    D = x.shape[-1]
    out = x if out is None else out
    _check("dsa_indexer_rope", lib().dsa_indexer_rope(
        _ptr(x), B, S, nh, D, rope_dim, _ptr(cos_t), _ptr(sin_t), cos_t.shape[0], _ptr(pos), _ptr(out),
        _stream(stream)))


def dsa_index_scores_fp8(q8, q_scale, k8, k_scale, w, seg, row0: int, nrows: int, scores, stream=None) -> None:
    B, S, Hi, Di = q8.shape
    ld = scores.shape[-1]
    _check("dsa_index_scores_fp8", lib().dsa_index_scores_fp8(
        _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(w), _ptr(seg), B, S, Hi, Di, row0, nrows,
        _ptr(scores), _dt(scores), ld, _stream(stream)))


def dsa_topk(scores, seg, B: int, S: int, K: int, row0: int, nrows: int, idx, mask, stream=None) -> None:
    ld = scores.shape[-1]
    _check("dsa_topk", lib().dsa_topk(
        _ptr(scores), _dt(scores), ld, _ptr(seg), B, S, K, row0, nrows, _ptr(idx), _ptr(mask),
        _stream(stream)))


def dsa_build_mask(idx, seg, mask, stream=None) -> None:
    B, S, K = idx.shape
    _check("dsa_build_mask", lib().dsa_build_mask(_ptr(idx), _ptr(seg), B, S, K, _ptr(mask),
                                                  _stream(stream)))


def dsa_sparse_attn_fwd(q, k, v, mask, softmax_scale: float, o, lse, stream=None) -> None:
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    _check("dsa_sparse_attn_fwd", lib().dsa_sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(mask), B, S, H, Dqk, Dv, float(softmax_scale), _dt(q),
        _ptr(o), _ptr(lse), _stream(stream)))


# compressed sparse attention: keys are Sk = S // ratio compressed entries
def dsa_csa_index_scores(q_idx, k_idx, w, ratio: int, row0: int, nrows: int, scores, stream=None) -> None:
    B, S, Hi, Di = q_idx.shape
    Sk = k_idx.shape[1]
    _check("dsa_csa_index_scores", lib().dsa_csa_index_scores(
        _ptr(q_idx), _ptr(k_idx), _ptr(w), B, S, Sk, ratio, Hi, Di, _dt(q_idx), row0, nrows, _ptr(scores),
        _dt(scores), scores.shape[-1], _stream(stream)))


def dsa_csa_topk(scores, B: int, S: int, Sk: int, ratio: int, K: int, row0: int, nrows: int, idx, mask,
                 stream=None) -> None:
    _check("dsa_csa_topk", lib().dsa_csa_topk(
        _ptr(scores), _dt(scores), scores.shape[-1], B, S, Sk, ratio, K, row0, nrows, _ptr(idx), _ptr(mask),
        _stream(stream)))


def dsa_csa_build_mask(idx, Sk: int, ratio: int, mask, stream=None) -> None:
    B, S, K = idx.shape
    _check("dsa_csa_build_mask", lib().dsa_csa_build_mask(_ptr(idx), B, S, Sk, ratio, K, _ptr(mask), _stream(stream)))


def dsa_csa_sparse_attn_fwd(q, k, v, mask, ratio: int, softmax_scale: float, o, lse, stream=None) -> None:
    B, S, H, Dqk = q.shape
    Sk, Dv = k.shape[1], v.shape[-1]
    _check("dsa_csa_sparse_attn_fwd", lib().dsa_csa_sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(mask), B, S, Sk, ratio, H, Dqk, Dv, float(softmax_scale), _dt(q), _ptr(o),
        _ptr(lse), _stream(stream)))


def dsa_csa_sparse_attn_bwd(q, k, v, o, dout, lse, mask, ratio: int, softmax_scale: float, dq, dk, dv, workspace,
                            stream=None) -> None:
    B, S, H, Dqk = q.shape
    Sk, Dv = k.shape[1], v.shape[-1]
    _check("dsa_csa_sparse_attn_bwd", lib().dsa_csa_sparse_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(mask), B, S, Sk, ratio, H, Dqk, Dv,
        float(softmax_scale), _dt(q), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def dsa_sparse_attn_bwd(q, k, v, o, dout, lse, mask, softmax_scale: float, dq, dk, dv, workspace,
                        stream=None) -> None:
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    _check("dsa_sparse_attn_bwd", lib().dsa_sparse_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(mask), B, S, H, Dqk, Dv,
        float(softmax_scale), _dt(q), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def dsa_sparse_attn_bwd_noalloc(q, k, v, o, dout, lse, mask, softmax_scale: float, dq, dk, dv,
                                stream=None) -> None:
    """dsa_sparse_attn_bwd with the library's own scratch array instead of a
    workspace (allocates nothing; calls overlapping on one GPU race)."""
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    _check("dsa_sparse_attn_bwd_noalloc", lib().dsa_sparse_attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(mask), B, S, H, Dqk, Dv,
        float(softmax_scale), _dt(q), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def dsa_sparse_attn_bwd_prep(o, dout, lse, Dqk: int, workspace, stream=None) -> None:
    """D and base-2 LSE into the workspace (first part of the backward)."""
    B, S, H, Dv = o.shape
    _check("dsa_sparse_attn_bwd_prep", lib().dsa_sparse_attn_bwd_prep(
        _ptr(o), _ptr(dout), _ptr(lse), B, S, H, Dqk, Dv, _dt(o), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def dsa_sparse_attn_bwd_dkdv(q, k, v, dout, lse, mask, softmax_scale: float, dk, dv, workspace,
                             stream=None) -> None:
    """Key-major part: dk, dv (and, on the MFMA path, the dS tiles for
    dsa_sparse_attn_bwd_dq); runs after dsa_sparse_attn_bwd_prep."""
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    _check("dsa_sparse_attn_bwd_dkdv", lib().dsa_sparse_attn_bwd_dkdv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(mask), B, S, H, Dqk, Dv,
        float(softmax_scale), _dt(q), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def dsa_sparse_attn_bwd_dq(q, k, v, dout, lse, mask, softmax_scale: float, dq, workspace,
                           stream=None) -> None:
    """Query-major half; runs after dsa_sparse_attn_bwd_dkdv on the same workspace."""
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    _check("dsa_sparse_attn_bwd_dq", lib().dsa_sparse_attn_bwd_dq(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(mask), B, S, H, Dqk, Dv,
        float(softmax_scale), _dt(q), _ptr(dq), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


# ------------------------------------------------------------------ indexer KL loss
def dsa_indexer_teacher(q, k, lse, mask, K: int, softmax_scale: float, teacher, stream=None) -> None:
    """teacher [B,S,K] float32: the head-averaged attention probabilities of
    each row's kept keys, in index-list order (0 past them)."""
    B, S, H, Dqk = q.shape
    _check("dsa_indexer_teacher", lib().dsa_indexer_teacher(
        _ptr(q), _ptr(k), _ptr(lse), _ptr(mask), B, S, H, Dqk, K, float(softmax_scale), _dt(q), _ptr(teacher),
        _stream(stream)))


def dsa_indexer_kl(scores, idx, teacher, mask, row_kl, loss, dscores, stream=None) -> None:
    """Student softmax over the kept scores, KL per row (row_kl [B,S]),
    loss = {mean KL, N} (float32[2]) and the score gradient dscores
    [B,S,ld_ds] float32 (over [0, t] of each row)."""
    B, S, K = idx.shape
    _check("dsa_indexer_kl", lib().dsa_indexer_kl(
        _ptr(scores), _dt(scores), scores.shape[-1], _ptr(idx), _ptr(teacher), _ptr(mask), B, S, K, _ptr(row_kl),
        _ptr(loss), _ptr(dscores), dscores.shape[-1], _stream(stream)))


def dsa_indexer_bwd(q_idx, k_idx, w, dscores, mask, dq_idx, dk_idx, dw, stream=None) -> None:
    """Gradients of sum(dscores * I) w.r.t. q_idx, k_idx and w."""
    B, S, Hi, Di = q_idx.shape
    _check("dsa_indexer_bwd", lib().dsa_indexer_bwd(
        _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(dscores), dscores.shape[-1], _ptr(mask), B, S, Hi, Di, _dt(q_idx),
        _ptr(dq_idx), _ptr(dk_idx), _ptr(dw), _stream(stream)))
