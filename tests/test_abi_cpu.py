"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (CPU only: no call here reaches a GPU)."""
import ctypes
import os
import re

import pytest
import torch

from sparse_attention_06_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="libdsa.so not built")

P = ctypes.c_void_p(0x10000)      # an aligned, never-dereferenced address
MIS = ctypes.c_void_p(0x10008)    # misaligned
NUL = None
S_ = ctypes.c_void_p(0)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|size_t|const char\*|int)\s+(dsa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(dsa.EXPORTS), names
    L = dsa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_sizes_and_strings():
    L = dsa.lib()
    B, S = 3, 1000
    W = (S + 63) // 64
    assert dsa.dsa_mask_bytes(B, S) == B * S * W * 8 + B * ((S + 127) // 128) * ((S + 63) // 64)
    assert dsa.dsa_mask_bytes(0, 5) == 0
    # D and base-2 LSE, rounded to 256 bytes; for the bf16 MFMA dims also the
    # dS tiles: each 32-query chunk c of a (b, h) holds key tiles 0..c//2, 4 KB each
    off = -(-(2 * 2 * 3 * 100 * 4) // 256) * 256
    assert dsa.dsa_bwd_workspace_min_bytes(2, 100, 3) == off
    assert dsa.dsa_bwd_workspace_bytes(2, 100, 3, 64, 64) == off
    assert dsa.dsa_bwd_workspace_bytes(2, 100, 3, 192, 128, torch.float32) == off   # plain path: no tiles
    tiles = sum(c // 2 + 1 for c in range((100 + 31) // 32))
    assert dsa.dsa_bwd_workspace_bytes(2, 100, 3, 192, 128) == off + 2 * 3 * tiles * 4096
    # the dS handoff is capped at 16 GiB: past it the recommended size is the
    # minimum (dQ recomputes dS), so memory stays linear in S
    cap = 16 << 30
    for B, S, H in ((12, 4096, 16), (4, 8192, 32), (1, 32768, 128), (1, 131072, 128)):
        t = sum(c // 2 + 1 for c in range((S + 31) // 32)) * 4096 * B * H
        want = dsa.dsa_bwd_workspace_min_bytes(B, S, H) + (t if t <= cap else 0)
        assert dsa.dsa_bwd_workspace_bytes(B, S, H, 192, 128) == want
    assert dsa.dsa_bwd_workspace_bytes(1, 32768, 128, 192, 128) == 8 * 32768 * 128
    assert dsa.dsa_bwd_workspace_min_bytes(0, 5, 1) == 0
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(3) == b"DSA_ERR_WORKSPACE"
    assert L.dsa_version() >= 100


def _idx_call(**kw):
    a = dict(q_idx=P, k_idx=P, w=P, seg=NUL, B=1, S=128, Hi=64, Di=128, dt=0, row0=0, nrows=128,
             scores=P, sdt=1, ld=128, st=S_)
    a.update(kw)
    return dsa.lib().dsa_index_scores(a["q_idx"], a["k_idx"], a["w"], a["seg"], a["B"], a["S"], a["Hi"],
                                      a["Di"], a["dt"], a["row0"], a["nrows"], a["scores"], a["sdt"],
                                      a["ld"], a["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(q_idx=NUL), 1), (dict(k_idx=MIS), 1), (dict(B=0), 1), (dict(S=-1), 1),
    (dict(row0=100, nrows=100), 1), (dict(ld=100), 1), (dict(dt=7), 1), (dict(seg=MIS), 1),
    (dict(Di=12), 2), (dict(Hi=4096, Di=64, dt=1), 2),
    # Hi * Di wraps a 32-bit int to a small value: still rejected (64-bit product)
    (dict(Hi=65536, Di=65535, dt=1), 2), (dict(Hi=65536, Di=65536, dt=1), 2),
    (dict(S=(1 << 18) + 1, nrows=1, ld=(1 << 18) + 1), 2),
])
def test_index_scores_rejects(kw, code):
    assert _idx_call(**kw) == code
    assert dsa.lib().dsa_last_error()


def _fp8_call(**kw):
    a = dict(q8=P, qs=P, k8=P, ks=P, w=P, seg=NUL, B=1, S=128, Hi=64, Di=128, row0=0, nrows=128,
             scores=P, sdt=1, ld=128, st=S_)
    a.update(kw)
    return dsa.lib().dsa_index_scores_fp8(a["q8"], a["qs"], a["k8"], a["ks"], a["w"], a["seg"], a["B"], a["S"],
                                          a["Hi"], a["Di"], a["row0"], a["nrows"], a["scores"], a["sdt"],
                                          a["ld"], a["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(q8=NUL), 1), (dict(ks=NUL), 1), (dict(k8=MIS), 1), (dict(B=0), 1), (dict(row0=100, nrows=100), 1),
    (dict(ld=100), 1), (dict(sdt=5), 1), (dict(Di=96), 2), (dict(Hi=48), 2), (dict(Hi=128), 2),
])
def test_index_scores_fp8_rejects(kw, code):
    assert _fp8_call(**kw) == code
    assert dsa.lib().dsa_last_error()


def test_quant_fp8_rejects():
    L = dsa.lib()
    assert L.dsa_quant_fp8_rows(NUL, 0, 4, 128, P, P, S_) == 1
    assert L.dsa_quant_fp8_rows(P, 0, 0, 128, P, P, S_) == 1
    assert L.dsa_quant_fp8_rows(P, 3, 4, 128, P, P, S_) == 1
    assert L.dsa_quant_fp8_rows(P, 0, 4, 96, P, P, S_) == 2
    assert L.dsa_quant_fp8_rows(MIS, 0, 4, 128, P, P, S_) == 1
    assert L.dsa_quant_fp8_rows(P, 0, 4, 128, MIS, P, S_) == 1
    assert L.dsa_quant_fp8_rows(P, 0, (1 << 26) + 1, 128, P, P, S_) == 2


def test_indexer_rope_rejects():
    L = dsa.lib()
    ok = (P, 2, 64, 4, 128, 64, P, P, 64, NUL, P, S_)
    assert L.dsa_indexer_rope(NUL, *ok[1:]) == 1
    assert L.dsa_indexer_rope(MIS, *ok[1:]) == 1
    assert L.dsa_indexer_rope(*ok[:8], 32, NUL, P, S_) == 1          # P < S without positions
    assert L.dsa_indexer_rope(*ok[:5], 40, *ok[6:]) == 2             # rope_dim % 16
    assert L.dsa_indexer_rope(*ok[:5], 144, *ok[6:]) == 2            # rope_dim > D
    assert L.dsa_indexer_rope(*ok[:4], 100, 64, *ok[6:]) == 2        # D % 8
    assert dsa.lib().dsa_last_error()


def test_topk_rejects():
    L = dsa.lib()
    # row slab not on a 128-row tile
    assert L.dsa_topk(P, 1, 300, NUL, 1, 300, 16, 64, 100, P, P, S_) == 1
    assert b"tile" in L.dsa_last_error()
    assert L.dsa_topk(P, 1, 300, NUL, 1, 300, 0, 0, 300, P, P, S_) == 1      # K = 0
    assert L.dsa_topk(NUL, 1, 300, NUL, 1, 300, 4, 0, 300, P, P, S_) == 1
    assert L.dsa_topk(P, 1, 299, NUL, 1, 300, 4, 0, 300, P, P, S_) == 1      # ld < S
    assert L.dsa_build_mask(P, MIS, 1, 10, 4, P, S_) == 1
    assert L.dsa_build_mask(P, NUL, 1, 10, 0, P, S_) == 1


def test_attention_rejects():
    L = dsa.lib()
    f32 = ctypes.c_float
    fwd = L.dsa_sparse_attn_fwd
    assert fwd(P, P, P, P, 1, 64, 2, 192, 128, f32(0.1), 0, P, NUL, S_) == 1         # lse NULL
    assert fwd(P, P, P, P, 1, 64, 2, 192, 128, f32(0.0), 0, P, P, S_) == 1           # scale 0
    assert fwd(P, P, P, P, 1, 64, 2, 512, 128, f32(0.1), 0, P, P, S_) == 2           # dim > 256
    assert fwd(P, P, P, P, 1, 64, 2, 100, 128, f32(0.1), 0, P, P, S_) == 2           # bf16 dim % 8
    bwd = L.dsa_sparse_attn_bwd
    need = dsa.dsa_bwd_workspace_min_bytes(1, 64, 2)
    assert bwd(P, P, P, P, P, P, P, 1, 64, 2, 192, 128, f32(0.1), 0, P, P, P, P, need - 4, S_) == 3
    assert b"workspace" in L.dsa_last_error()
    assert bwd(P, P, P, P, P, P, P, 1, 64, 2, 192, 128, f32(0.1), 0, P, P, MIS, P, need, S_) == 1


def test_noalloc_backward_rejects_before_any_launch():
    L = dsa.lib()
    f32 = ctypes.c_float
    na = L.dsa_sparse_attn_bwd_noalloc
    assert na(P, P, P, P, P, P, NUL, 1, 64, 2, 192, 128, f32(0.1), 0, P, P, P, S_) == 1     # mask NULL
    assert na(P, P, P, P, P, P, P, 1, 64, 2, 192, 128, f32(0.1), 0, P, MIS, P, S_) == 1     # misaligned dk
    assert na(P, P, P, P, P, P, P, 1, 64, 2, 512, 128, f32(0.1), 0, P, P, P, S_) == 2       # dim > 256
    # 8 bytes per (b, h, t) must fit the 64 MiB scratch: B*H*S <= 8 Mi
    assert na(P, P, P, P, P, P, P, 1, 1 << 18, 33, 192, 128, f32(0.1), 0, P, P, P, S_) == 2
    assert b"scratch" in L.dsa_last_error()
    assert na(P, P, P, P, P, P, P, 2, 65536, 65, 192, 128, f32(0.1), 0, P, P, P, S_) == 2


def test_indexer_loss_calls_reject_before_any_launch():
    L = dsa.lib()
    f32 = ctypes.c_float
    # teacher: bf16 only, Dqk in {64, 128, 192}
    assert L.dsa_indexer_teacher(P, P, P, P, 1, 64, 2, 192, 16, f32(0.1), 1, P, S_) == 2
    assert L.dsa_indexer_teacher(P, P, P, P, 1, 64, 2, 96, 16, f32(0.1), 0, P, S_) == 2
    assert L.dsa_indexer_teacher(P, P, P, P, 1, 64, 2, 192, 0, f32(0.1), 0, P, S_) == 1
    assert L.dsa_indexer_teacher(P, P, NUL, P, 1, 64, 2, 192, 16, f32(0.1), 0, P, S_) == 1
    # kl: loss must be an 8-byte aligned float[2]; ld >= S
    kl = L.dsa_indexer_kl
    assert kl(P, 1, 64, P, P, P, 1, 64, 16, P, ctypes.c_void_p(0x10004), P, 64, S_) == 1
    assert kl(P, 1, 63, P, P, P, 1, 64, 16, P, P, P, 64, S_) == 1
    assert kl(P, 1, 64, P, P, P, 1, 64, 16, P, P, P, 60, S_) == 1
    # bwd: 64 x 128 bf16, ld >= S
    bw = L.dsa_indexer_bwd
    assert bw(P, P, P, P, 64, P, 1, 64, 32, 128, 0, P, P, P, S_) == 2
    assert bw(P, P, P, P, 64, P, 1, 64, 64, 64, 0, P, P, P, S_) == 2
    assert bw(P, P, P, P, 63, P, 1, 64, 64, 128, 0, P, P, P, S_) == 1
    assert bw(P, P, P, P, 64, P, 1, 64, 64, 128, 1, P, P, P, S_) == 2


def test_csa_sizes_and_rejects():
    """Compressed-key calls: mask size over Sk keys; ratio, Sk and ld checked
    on the host before any launch."""
    L = dsa.lib()
    B, S, Sk = 2, 1000, 250
    W = (Sk + 63) // 64
    assert dsa.dsa_csa_mask_bytes(B, S, Sk) == B * S * W * 8 + B * ((S + 127) // 128) * ((Sk + 63) // 64)
    assert dsa.dsa_csa_mask_bytes(B, S, S) == dsa.dsa_mask_bytes(B, S)
    assert dsa.dsa_csa_mask_bytes(B, S, 0) == 0

    def scores(**kw):
        a = dict(B=1, S=128, Sk=32, r=4, ld=32, row0=0, nrows=128)
        a.update(kw)
        return L.dsa_csa_index_scores(P, P, P, a["B"], a["S"], a["Sk"], a["r"], 64, 128, 0, a["row0"], a["nrows"],
                                      P, 1, a["ld"], S_)

    for kw in (dict(r=0), dict(Sk=33), dict(Sk=31), dict(S=3, Sk=0, nrows=3), dict(ld=31), dict(nrows=129)):
        assert scores(**kw) == 1, kw

    def topk(**kw):
        a = dict(S=128, Sk=32, r=4, K=8, ld=32, row0=0, nrows=128)
        a.update(kw)
        return L.dsa_csa_topk(P, 0, a["ld"], 1, a["S"], a["Sk"], a["r"], a["K"], a["row0"], a["nrows"], P, P, S_)

    for kw in (dict(r=-1), dict(Sk=64), dict(K=0), dict(ld=16), dict(row0=64, nrows=64)):
        assert topk(**kw) == 1, kw
    assert L.dsa_csa_build_mask(P, 1, 128, 64, 4, 8, P, S_) == 1       # Sk != S / ratio
    assert L.dsa_csa_build_mask(NUL, 1, 128, 32, 4, 8, P, S_) == 1
    fwd = L.dsa_csa_sparse_attn_fwd
    assert fwd(P, P, P, P, 1, 128, 32, 0, 2, 192, 128, 0.1, 0, P, P, S_) == 1      # ratio 0
    assert fwd(P, P, P, P, 1, 128, 31, 4, 2, 192, 128, 0.1, 0, P, P, S_) == 1      # Sk
    assert fwd(P, P, P, P, 1, 128, 32, 4, 2, 192, 128, -1.0, 0, P, P, S_) == 1     # scale
    assert fwd(P, P, P, MIS, 1, 128, 32, 4, 2, 192, 128, 0.1, 0, P, P, S_) == 1    # misaligned mask
    assert fwd(P, P, P, P, 1, 128, 32, 4, 2, 512, 128, 0.1, 0, P, P, S_) == 2      # head dim above 256


def test_csa_backward_rejects_before_any_launch():
    bwd = dsa.lib().dsa_csa_sparse_attn_bwd
    need = dsa.dsa_bwd_workspace_min_bytes(1, 128, 2)
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", P), ("k", P), ("v", P), ("o", P), ("dout", P), ("lse", P), ("mask", P), ("B", 1), ("S", 128),
        ("Sk", 32), ("r", 4), ("H", 2), ("Dqk", 192), ("Dv", 128), ("scale", 0.1), ("dt", 0), ("dq", P), ("dk", P),
        ("dv", P), ("ws", P), ("wsb", need), ("st", S_))]
    assert bwd(*args(r=0)) == 1
    assert bwd(*args(Sk=33)) == 1
    assert bwd(*args(dk=NUL)) == 1
    assert bwd(*args(mask=MIS)) == 1
    assert bwd(*args(wsb=need - 1)) == 3      # DSA_ERR_WORKSPACE
    assert bwd(*args(Dqk=300)) == 2


def test_csa_backward_workspace_sizes():
    B, S, Sk, r, H = 2, 1000, 250, 4, 3
    base = dsa.dsa_bwd_workspace_min_bytes(B, S, H)
    nch, nkt = (S + 31) // 32, (Sk + 63) // 64
    assert dsa.dsa_csa_bwd_workspace_bytes(B, S, Sk, r, H, 192, 128) == base + B * H * nch * nkt * 4096
    assert dsa.dsa_csa_bwd_workspace_bytes(B, S, Sk, r, H, 64, 64) == base                 # plain kernels
    assert dsa.dsa_csa_bwd_workspace_bytes(B, S, S, 1, H, 192, 128) == dsa.dsa_bwd_workspace_bytes(B, S, H, 192, 128)
    assert dsa.dsa_csa_bwd_workspace_bytes(B, S, 0, r, H, 192, 128) == 0
