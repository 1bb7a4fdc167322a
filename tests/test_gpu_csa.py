"""Parity of the compressed-key (CSA) forward path with the float64 oracle.

Keys are Sk = S // ratio compressed entries; entry c is visible to query t
when ratio*c + ratio - 1 <= t. Small shapes are checked element by element
(several tiles, a ragged tail, the rows before the first complete block);
long rows take the single-read and multi-pass top-k kernels; the CSA workload
runs at full size with sampled rows. Index sets for the attention tests are
token-level random sets mapped to their blocks (c = s // ratio), so they mix
visible entries, entries of the row's own incomplete block and duplicates,
which the mask builder must drop or merge.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, check_undecidable_row, f64, row_decision
from oracle import dsa_oracle as ref
from sparse_attention_06_amd import dsa, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _cfg(**kw):
    return inputs.CSA_CONFIGS["csa"].replace(B=2, S=333, H=3, K=16).replace(**kw)


def _make(cfg):
    x = inputs.make(cfg, device="cpu")
    return x, {k: v.to(DEV).contiguous() for k, v in x.items() if v is not None}


def _keys(scores_f64, valid_rows):
    return np.where(valid_rows, scores_f64, -np.inf)


def _valid(Sk, ratio, rows):
    return np.stack([ref.csa_valid_row(Sk, ratio, int(t)) for t in rows])


def _check_scores(got, want, bf16):
    fin = np.isfinite(want)
    assert np.all(np.isfinite(got[fin]))
    rowmax = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
    err = np.abs(np.where(fin, got - want, 0))
    if bf16:
        ulp = np.ldexp(1.0, np.frexp(np.abs(np.where(fin, want, 1.0)))[1] - 8)
        assert np.all(err <= ulp + 1e-6 * rowmax), err.max()
    else:
        assert np.all(err <= 1e-5 * rowmax + 1e-7), err.max()


def _check_mask(mask, idx_np, B, S, Sk):
    M = ref.selection_matrix(idx_np, Sk)
    bits, cls = dsa.mask_views(mask, B, S, Sk)
    assert np.array_equal(bits.cpu().numpy(), ref.pack_bits(M).view(np.int64))
    assert np.array_equal(cls.cpu().numpy(), ref.tile_classes(M, 128, 64))


# ------------------------------------------------------------------ indexer + top-k + mask
@pytest.mark.parametrize("ratio", [4, 3])
@pytest.mark.parametrize("score_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("HiDi,dtype", [((64, 128), "bf16"), ((4, 32), "fp32")])
def test_csa_indexer_topk_mask(ratio, score_dtype, HiDi, dtype):
    Hi, Di = HiDi
    cfg = _cfg(ratio=ratio, Hi=Hi, Di=Di, dtype=dtype)
    x, d = _make(cfg)
    B, S, Sk, K = cfg.B, cfg.S, cfg.Sk, cfg.K
    sc = torch.full((B, S, Sk), float("nan"), dtype=score_dtype, device=DEV)
    dsa.dsa_csa_index_scores(d["q_idx"], d["k_idx"], d["w"], ratio, 0, S, sc)
    idx = torch.full((B, S, K), -7, dtype=torch.int32, device=DEV)
    mask = torch.full((dsa.dsa_csa_mask_bytes(B, S, Sk),), 0xAB, dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_topk(sc, B, S, Sk, ratio, K, 0, S, idx, mask)
    torch.cuda.synchronize()
    rows = np.arange(S)
    want = ref.csa_index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), ratio, rows)
    got = f64(sc)
    _check_scores(got, want, score_dtype == torch.bfloat16)
    valid = _valid(Sk, ratio, rows)[None]
    # on the GPU's own keys the selection is unique: exact, masks from the lists
    own = ref.csa_topk(_keys(got, valid), ratio, rows, K, Sk)
    gidx = idx.cpu().numpy()
    assert np.array_equal(gidx, own)
    _check_mask(mask, own, B, S, Sk)
    assert np.all(gidx[:, : ratio - 1] == -1)  # rows before the first complete block keep nothing
    # against the oracle's own selection: exact on decidable rows
    keys_ref = ref.bf16_round(want) if score_dtype == torch.bfloat16 else want
    want_idx = ref.csa_topk(keys_ref, ratio, rows, K, Sk)
    n_dec = 0
    for b in range(B):
        for t in rows:
            v = valid[0, t]
            dec, k_n, k_n1, tau = row_decision(keys_ref[b, t], got[b, t], v, K)
            if dec:
                assert np.array_equal(gidx[b, t], want_idx[b, t]), (b, t)
                n_dec += 1
            else:
                check_undecidable_row(keys_ref[b, t], v, gidx[b, t], K, k_n, k_n1, tau)
    assert n_dec >= 0.75 * B * S


def test_csa_ratio_one_is_dsa_bit_for_bit():
    """The compressed-key calls with ratio 1 give the token-level calls' bits."""
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, H=3, K=64)
    x, d = _make(cfg)
    B, S, K = cfg.B, cfg.S, cfg.K
    outs = []
    for csa in (False, True):
        sc = torch.zeros((B, S, S), dtype=torch.float32, device=DEV)
        idx = torch.empty((B, S, K), dtype=torch.int32, device=DEV)
        mask = torch.empty(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
        o = torch.empty((B, S, cfg.H, cfg.Dv), dtype=d["q"].dtype, device=DEV)
        lse = torch.empty((B, cfg.H, S), dtype=torch.float32, device=DEV)
        if csa:
            dsa.dsa_csa_index_scores(d["q_idx"], d["k_idx"], d["w"], 1, 0, S, sc)
            dsa.dsa_csa_topk(sc, B, S, S, 1, K, 0, S, idx, mask)
            dsa.dsa_csa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, 1, cfg.softmax_scale, o, lse)
        else:
            dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], None, 0, S, sc)
            dsa.dsa_topk(sc, None, B, S, K, 0, S, idx, mask)
            dsa.dsa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, cfg.softmax_scale, o, lse)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (sc, idx, mask, o, lse)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# ------------------------------------------------------------------ attention
def _entry_sets(cfg):
    """Token-level random sets mapped to their blocks: int32 [B, S, K]."""
    tok = inputs.random_index_sets(cfg.B, cfg.S, cfg.K, None, seed=11)
    return np.where(tok >= 0, tok // cfg.ratio, -1).astype(np.int32)


@pytest.mark.parametrize("ratio,dims,dtype", [(4, (192, 128), "bf16"), (3, (192, 128), "bf16"),
                                              (4, (64, 64), "fp32"), (5, (64, 32), "bf16")])
def test_csa_build_mask_and_attention_fwd(ratio, dims, dtype):
    cfg = _cfg(ratio=ratio, Dqk=dims[0], Dv=dims[1], dtype=dtype, K=24)
    x, d = _make(cfg)
    B, S, Sk, H = cfg.B, cfg.S, cfg.Sk, cfg.H
    sets = _entry_sets(cfg)
    mask = torch.full((dsa.dsa_csa_mask_bytes(B, S, Sk),), 0x5A, dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_build_mask(torch.from_numpy(sets).to(DEV), Sk, ratio, mask)
    o = torch.full((B, S, H, cfg.Dv), float("nan"), dtype=d["q"].dtype, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, ratio, cfg.softmax_scale, o, lse)
    torch.cuda.synchronize()
    # the mask holds the visible entries of each set, nothing else
    vis = _valid(Sk, ratio, np.arange(S))
    kept = np.full_like(sets, -1)
    for b in range(B):
        for t in range(S):
            e = np.unique(sets[b, t][(sets[b, t] >= 0) & (sets[b, t] < Sk)])
            e = e[vis[t, e]]
            kept[b, t, : e.size] = e
    _check_mask(mask, kept, B, S, Sk)
    O, L = ref.csa_attention_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), sets, ratio, cfg.softmax_scale,
                                 np.arange(S))
    bf16 = dtype == "bf16"
    check_close("O", f64(o), O, bf16)
    lg = lse.cpu().numpy()
    assert np.array_equal(np.isinf(lg), np.isinf(L))
    fin = np.isfinite(L)
    np.testing.assert_allclose(lg[fin], L[fin], rtol=0, atol=1e-4 if bf16 else 1e-5)
    empty = ~(kept >= 0).any(axis=-1)          # [B, S]
    assert empty[:, : ratio - 1].all()
    assert np.all(f64(o)[empty] == 0)


# ------------------------------------------------------------------ long rows
@pytest.mark.parametrize("K", [512, 3500])
def test_csa_topk_long_rows(K):
    """Rows with more than 4096 visible entries: the single-read kernel (K =
    512) and the multi-pass kernel (K = 3500), exact on the GPU's keys."""
    B, S, ratio = 1, 17000, 4
    Sk = S // ratio
    cfg = _cfg(B=B, S=S, ratio=ratio, K=K)
    x, d = _make(cfg)
    sc = torch.empty((B, S, Sk), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_index_scores(d["q_idx"], d["k_idx"], d["w"], ratio, 0, S, sc)
    idx = torch.empty((B, S, K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_csa_mask_bytes(B, S, Sk), dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_topk(sc, B, S, Sk, ratio, K, 0, S, idx, mask)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(S - 4, S), [16386, 16387, 16388, 16391, 2047, 0, 3],
                                     rng.integers(16387, S, 24), rng.integers(0, S, 8)]))
    got = f64(sc[:, torch.from_numpy(rows).to(DEV)])
    valid = _valid(Sk, ratio, rows)[None]
    own = ref.csa_topk(_keys(got, valid), ratio, rows, K, Sk)
    assert np.array_equal(idx.cpu().numpy()[:, rows], own)
    bits, _ = dsa.mask_views(mask, B, S, Sk)
    M = ref.selection_matrix(own, Sk)
    assert np.array_equal(bits.cpu().numpy()[:, rows], ref.pack_bits(M).view(np.int64))
    # the scores of those rows against the oracle, row by row
    k_b = f64(x["k_idx"][0])
    want = np.stack([ref.index_scores_row(f64(x["q_idx"][0, t]), f64(x["w"][0, t]), k_b,
                                          ref.csa_valid_row(Sk, ratio, int(t))) for t in rows])[None]
    _check_scores(got, want, False)


# ------------------------------------------------------------------ the CSA workload at full size
def test_csa_workload_fullsize():
    """The CSA workload (B=12, S=4096, ratio 4, K=512, 16 heads of 192/128):
    indexer, top-k and forward on the GPU; sampled rows against the oracle."""
    cfg = inputs.CSA_CONFIGS["csa"]
    x = inputs.make(cfg, device=DEV)
    B, S, Sk, K, H = cfg.B, cfg.S, cfg.Sk, cfg.K, cfg.H
    sc = torch.empty((B, S, Sk), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, S, K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_csa_mask_bytes(B, S, Sk), dtype=torch.uint8, device=DEV)
    o = torch.empty((B, S, H, cfg.Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_index_scores(x["q_idx"], x["k_idx"], x["w"], cfg.ratio, 0, S, sc)
    dsa.dsa_csa_topk(sc, B, S, Sk, cfg.ratio, K, 0, S, idx, mask)
    dsa.dsa_csa_sparse_attn_fwd(x["q"], x["k"], x["v"], mask, cfg.ratio, cfg.softmax_scale, o, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(S - 8, S), [4 * K - 2, 4 * K - 1, 4 * K, 4 * K + 3],
                                     rng.integers(0, S, 64)]))
    n_dec = 0
    for b in (0, B - 1):
        k_b = f64(x["k_idx"][b])
        for t in rows:
            t = int(t)
            valid = ref.csa_valid_row(Sk, cfg.ratio, t)
            rs = ref.index_scores_row(f64(x["q_idx"][b, t]), f64(x["w"][b, t]), k_b, valid)
            g = f64(sc[b, t])
            fin = valid
            assert np.all(np.abs(g[fin] - rs[fin]) <= 1e-5 * np.abs(rs[fin]).max(initial=0) + 1e-7), (b, t)
            gi = idx[b, t].cpu().numpy()
            own = ref.topk_row(np.where(valid, g, -np.inf), valid, K)
            assert np.array_equal(gi[: own.size], own) and np.all(gi[own.size:] == -1), (b, t)
            dec, k_n, k_n1, tau = row_decision(rs, g, valid, K)
            sel = ref.topk_row(rs, valid, K)
            if dec:
                assert np.array_equal(own, sel), (b, t)
                n_dec += 1
            else:
                check_undecidable_row(rs, valid, gi, K, k_n, k_n1, tau)
                sel = own
            if sel.size == 0:
                assert np.all(f64(o[b, t]) == 0) and np.all(np.isinf(lse[b, :, t].cpu().numpy()))
                continue
            Ot, Lt = ref.attention_fwd_row(f64(x["q"][b, t]), f64(x["k"][b, torch.from_numpy(sel).to(DEV)]),
                                           f64(x["v"][b, torch.from_numpy(sel).to(DEV)]), cfg.softmax_scale)
            check_close(f"O[{b},{t}]", f64(o[b, t]), Ot, True)
            np.testing.assert_allclose(lse[b, :, t].cpu().numpy(), Lt, rtol=0, atol=1e-4)
    assert n_dec >= 0.75 * 2 * rows.size


# ------------------------------------------------------------------ backward
@pytest.mark.parametrize("ratio,dims,dtype,handoff", [(4, (192, 128), "bf16", True), (4, (192, 128), "bf16", False),
                                                      (3, (192, 128), "bf16", True), (3, (64, 64), "fp32", False),
                                                      (5, (64, 32), "bf16", False)])
def test_csa_attention_bwd(ratio, dims, dtype, handoff):
    """dq, dk, dv of the compressed keys, element by element, on mapped random
    sets (visible entries, incomplete blocks, duplicates, past-the-end
    entries), after the forward on the same mask. bf16 192/128 takes the MFMA
    kernels, with the dS handoff (workspace of dsa_csa_bwd_workspace_bytes) or
    without it (the minimum workspace: dQ from the MFMA kernel that recomputes
    dS)."""
    cfg = _cfg(ratio=ratio, Dqk=dims[0], Dv=dims[1], dtype=dtype, K=24, backward=True)
    x, d = _make(cfg)
    B, S, Sk, H = cfg.B, cfg.S, cfg.Sk, cfg.H
    sets = _entry_sets(cfg)
    mask = torch.empty(dsa.dsa_csa_mask_bytes(B, S, Sk), dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_build_mask(torch.from_numpy(sets).to(DEV), Sk, ratio, mask)
    o = torch.empty((B, S, H, cfg.Dv), dtype=d["q"].dtype, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, ratio, cfg.softmax_scale, o, lse)
    dq = torch.full_like(d["q"], float("nan"))
    dk = torch.full_like(d["k"], float("nan"))
    dv = torch.full_like(d["v"], float("nan"))
    nws = (dsa.dsa_csa_bwd_workspace_bytes(B, S, Sk, ratio, H, cfg.Dqk, cfg.Dv, d["q"].dtype) if handoff
           else dsa.dsa_bwd_workspace_min_bytes(B, S, H))
    ws = torch.full((nws,), 0x7F, dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, mask, ratio, cfg.softmax_scale, dq, dk,
                                dv, ws)
    torch.cuda.synchronize()
    want_dq, want_dk, want_dv = ref.csa_attention_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), sets,
                                                      ratio, cfg.softmax_scale)
    bf16 = dtype == "bf16"
    rel = 2e-2 if bf16 else None
    check_close("dq", f64(dq), want_dq, bf16, rel)
    check_close("dk", f64(dk), want_dk, bf16, rel)
    check_close("dv", f64(dv), want_dv, bf16, rel)
    assert np.all(f64(dq)[:, : ratio - 1] == 0)   # rows that see no entry


@pytest.mark.parametrize("ratio,S", [(4, 333), (3, 700)])
def test_csa_bwd_recompute_route_matches_handoff(ratio, S):
    """Over compressed keys the two dQ routes of the MFMA backward (dS handed
    over by the key-major kernel, or recomputed by the query-major one) give
    the same bits, and dK/dV do not depend on the route."""
    cfg = _cfg(ratio=ratio, S=S, K=40, backward=True)
    x, d = _make(cfg)
    B, Sk, H = cfg.B, cfg.Sk, cfg.H
    sets = _entry_sets(cfg)
    mask = torch.empty(dsa.dsa_csa_mask_bytes(B, S, Sk), dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_build_mask(torch.from_numpy(sets).to(DEV), Sk, ratio, mask)
    o = torch.empty((B, S, H, cfg.Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, ratio, cfg.softmax_scale, o, lse)
    outs = []
    for nws in (dsa.dsa_csa_bwd_workspace_bytes(B, S, Sk, ratio, H, cfg.Dqk, cfg.Dv),
                dsa.dsa_bwd_workspace_min_bytes(B, S, H)):
        g = [torch.full_like(d[n], float("nan")) for n in ("q", "k", "v")]
        ws = torch.full((nws,), 0x7F, dtype=torch.uint8, device=DEV)
        dsa.dsa_csa_sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, mask, ratio, cfg.softmax_scale,
                                    *g, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in g])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint16), b.view(torch.uint16))


def test_csa_bwd_ratio_one_is_dsa_bit_for_bit():
    """The compressed-key backward with ratio 1 (MFMA, dS handoff) gives the
    token-level backward's bits."""
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, H=3, K=64)
    x, d = _make(cfg)
    B, S, H, K = cfg.B, cfg.S, cfg.H, cfg.K
    sets = torch.from_numpy(inputs.random_index_sets(B, S, K, None, seed=2)).to(DEV)
    mask = torch.empty(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    dsa.dsa_build_mask(sets, None, mask)
    o = torch.empty((B, S, H, cfg.Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_attn_fwd(d["q"], d["k"], d["v"], mask, cfg.softmax_scale, o, lse)
    nws = dsa.dsa_bwd_workspace_bytes(B, S, H, cfg.Dqk, cfg.Dv)
    assert nws == dsa.dsa_csa_bwd_workspace_bytes(B, S, S, 1, H, cfg.Dqk, cfg.Dv)
    outs = []
    for csa in (False, True):
        g = [torch.empty_like(d[n]) for n in ("q", "k", "v")]
        ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
        if csa:
            dsa.dsa_csa_sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, mask, 1, cfg.softmax_scale, *g, ws)
        else:
            dsa.dsa_sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, mask, cfg.softmax_scale, *g, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in g])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_csa_bwd_fullsize():
    """The CSA workload's backward (MFMA, dS handoff) on the selection the
    forward path makes: sampled dQ rows, every element of dK/dV for the last
    64 entries of one head (only rows t >= S - 256 see them), and the sum
    rules over all entries."""
    cfg = inputs.CSA_CONFIGS["csa"].replace(backward=True)
    x = inputs.make(cfg, device=DEV)
    B, S, Sk, K, H, r = cfg.B, cfg.S, cfg.Sk, cfg.K, cfg.H, cfg.ratio
    sc = torch.empty((B, S, Sk), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, S, K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_csa_mask_bytes(B, S, Sk), dtype=torch.uint8, device=DEV)
    o = torch.empty((B, S, H, cfg.Dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    dsa.dsa_csa_index_scores(x["q_idx"], x["k_idx"], x["w"], r, 0, S, sc)
    dsa.dsa_csa_topk(sc, B, S, Sk, r, K, 0, S, idx, mask)
    dsa.dsa_csa_sparse_attn_fwd(x["q"], x["k"], x["v"], mask, r, cfg.softmax_scale, o, lse)
    dq, dk, dv = (torch.empty_like(x[n]) for n in ("q", "k", "v"))
    ws = torch.empty(dsa.dsa_csa_bwd_workspace_bytes(B, S, Sk, r, H, cfg.Dqk, cfg.Dv), dtype=torch.uint8, device=DEV)
    dsa.dsa_csa_sparse_attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, mask, r, cfg.softmax_scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    b = B - 1
    gidx = idx[b].cpu().numpy()
    rng = np.random.default_rng(9)
    for t in np.unique(np.concatenate([[0, 3, 4, 2047, 2051, S - 1], rng.integers(0, S, 24)])):
        t = int(t)
        sel = gidx[t][gidx[t] >= 0].astype(np.int64)
        if sel.size == 0:
            assert np.all(f64(dq[b, t]) == 0)
            continue
        g = lambda n: f64(x[n][b, torch.from_numpy(sel).to(DEV)])
        dq_t, _, _ = ref.attention_bwd_row(f64(x["q"][b, t]), g("k"), g("v"), f64(x["dout"][b, t]), cfg.softmax_scale)
        check_close(f"dq[{b},{t}]", f64(dq[b, t]), dq_t, True, 2e-2)
    # the last 64 entries of head h: rows t >= r * (Sk - 64) + r - 1 see them
    h, c0 = H // 2, Sk - 64
    rows = np.arange(r * c0 + r - 1, S)
    sl = slice(h, h + 1)
    want_dk = np.zeros((64, cfg.Dqk))
    want_dv = np.zeros((64, cfg.Dv))
    qh, doh = f64(x["q"][b, :, sl]), f64(x["dout"][b, :, sl])
    kh, vh = f64(x["k"][b, :, sl]), f64(x["v"][b, :, sl])
    for t in rows:
        sel = gidx[t][gidx[t] >= 0].astype(np.int64)
        _, dks, dvs = ref.attention_bwd_row(qh[t], kh[sel], vh[sel], doh[t], cfg.softmax_scale)
        late = sel >= c0
        want_dk[sel[late] - c0] += dks[late, 0]
        want_dv[sel[late] - c0] += dvs[late, 0]
    check_close("dk tail", f64(dk[b, c0:, h]), want_dk, True, 2e-2)
    check_close("dv tail", f64(dv[b, c0:, h]), want_dv, True, 2e-2)
    # sum rules: sum_c dK(c) = 0; sum_c dV(c) = sum of dO over the rows that keep an entry
    dks = dk.float().sum(dim=1)
    assert torch.all(dks.abs() <= 1e-2 * dk.float().abs().sum(dim=1) + 1e-3)
    live = torch.from_numpy(np.arange(S) >= r - 1).to(DEV)
    dvs = dv.float().sum(dim=1)
    do = (x["dout"].float() * live[None, :, None, None]).sum(dim=1)
    assert torch.all((dvs - do).abs() <= 1e-2 * dv.float().abs().sum(dim=1) + 1e-2)
