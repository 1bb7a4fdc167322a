"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Sizes here are ones the oracle finishes in seconds, spanning several tiles
and a ragged tail. The full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from gpu_util import (check_close, compare_topk_rows, f64)
from oracle import dsa_oracle as ref
from sparse_attention_06_amd import dsa, inputs
from sparse_attention_06_amd.pipeline import DSAPath

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _cfg(**kw):
    base = inputs.CONFIGS["c2"].replace(B=2, S=333, H=3, K=64, backward=True)
    return base.replace(**kw)


def _seg_np(x):
    return None if x["seg"] is None else x["seg"].cpu().numpy()


def _seg_dev(x):
    return None if x["seg"] is None else x["seg"].to(DEV).contiguous()


def _make(cfg, device=DEV):
    x = inputs.make(cfg, device="cpu")
    return x, {k: (None if v is None else v.to(device).contiguous()) for k, v in x.items()}


# ------------------------------------------------------------------ indexer
@pytest.mark.parametrize("segments", [None, (40, 150)])
@pytest.mark.parametrize("score_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("HiDi", [(64, 128), (32, 64)])
def test_indexer_mfma_parity(segments, score_dtype, HiDi):
    Hi, Di = HiDi
    cfg = _cfg(Hi=Hi, Di=Di, segments=segments)
    x, d = _make(cfg)
    S = cfg.S
    sc = torch.full((cfg.B, S, S), float("nan"), dtype=score_dtype, device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], _seg_dev(x), 0, S, sc)
    torch.cuda.synchronize()
    rows = np.arange(S)
    want = ref.index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), _seg_np(x), rows)
    got = f64(sc)
    fin = np.isfinite(want)
    assert np.all(np.isfinite(got[fin]))
    rowmax = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
    err = np.abs(np.where(fin, got - want, 0))
    if score_dtype == torch.float32:
        assert np.all(err <= 1e-5 * rowmax + 1e-7), err.max()
    else:
        # one bf16 rounding of the float32 score: within one bf16 ulp of the exact value
        ulp = np.ldexp(1.0, np.frexp(np.abs(np.where(fin, want, 1.0)))[1] - 8)
        assert np.all(err <= ulp + 1e-6 * rowmax), err.max()


@pytest.mark.parametrize("dtype,Hi,Di", [("fp32", 4, 32), ("bf16", 48, 40), ("fp32", 64, 128)])
def test_indexer_plain_parity(dtype, Hi, Di):
    cfg = _cfg(Hi=Hi, Di=Di, dtype=dtype, scaled=dtype == "bf16", S=200)
    x, d = _make(cfg)
    S = cfg.S
    sc = torch.zeros((cfg.B, S, S), dtype=torch.float32, device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], None, 0, S, sc)
    torch.cuda.synchronize()
    want = ref.index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), None, np.arange(S))
    fin = np.isfinite(want)
    rowmax = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
    err = np.abs(np.where(fin, f64(sc) - want, 0))
    assert np.all(err <= 1e-5 * rowmax + 1e-6), err.max()


def test_indexer_slabs_match_whole_call():
    cfg = _cfg(segments=(30, 120))
    x, d = _make(cfg)
    S = cfg.S
    whole = torch.zeros((cfg.B, S, S), device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], _seg_dev(x), 0, S, whole)
    buf = torch.zeros(cfg.B * 128 * S, device=DEV)
    valid = torch.from_numpy(np.stack([np.stack([ref.valid_row(_seg_np(x)[b], S, t) for t in range(S)])
                                       for b in range(cfg.B)])).to(DEV)
    for row0 in range(0, S, 128):
        n = min(128, S - row0)
        part = buf[: cfg.B * n * S].view(cfg.B, n, S)      # [B, nrows, ld] for this slab
        dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], _seg_dev(x), row0, n, part)
        v = valid[:, row0:row0 + n]
        assert torch.equal(part[v], whole[:, row0:row0 + n][v])


# ------------------------------------------------------------------ top-k
def _mask_ref(idx_np, S):
    M = ref.selection_matrix(idx_np, S)
    return ref.pack_bits(M).view(np.int64), ref.tile_classes(M, 128, 64)


@pytest.mark.parametrize("S,K,segments,score_dtype", [
    (700, 64, None, torch.float32), (700, 64, (50, 300), torch.float32),
    (300, 512, None, torch.float32), (513, 1, None, torch.float32),
    (700, 100, None, torch.bfloat16), (1000, 200, (64, 500), torch.bfloat16)])
def test_topk_exact_on_gpu_scores(S, K, segments, score_dtype):
    """Given identical keys the selection is unique: GPU == oracle bit for bit."""
    cfg = _cfg(S=S, K=K, segments=segments)
    x, d = _make(cfg)
    B = cfg.B
    sc = torch.zeros((B, S, S), dtype=score_dtype, device=DEV)
    idx = torch.empty((B, S, K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["k_idx"], d["w"], _seg_dev(x), 0, S, sc)
    dsa.dsa_topk(sc, _seg_dev(x), B, S, K, 0, S, idx, mask)
    torch.cuda.synchronize()
    keys = f64(sc)
    want = ref.topk(keys, _seg_np(x), np.arange(S), K, S)
    assert np.array_equal(idx.cpu().numpy(), want)
    bits, cls = dsa.mask_views(mask, B, S)
    wb, wc = _mask_ref(want, S)
    assert np.array_equal(bits.cpu().numpy(), wb)
    assert np.array_equal(cls.cpu().numpy(), wc)


def test_topk_ties_and_signed_zeros():
    """Crafted scores with heavy ties, -0/+0, and slab calls."""
    B, S, K = 2, 640, 37
    g = torch.Generator().manual_seed(5)
    vals = (torch.randint(-4, 5, (B, S, S), generator=g).float() * 0.25)
    vals[torch.rand((B, S, S), generator=g) < 0.05] = -0.0
    vals[:, 200:300] = 0.0                         # whole rows of zeros
    sc = vals.to(DEV)
    idx = torch.full((B, S, K), -7, dtype=torch.int32, device=DEV)
    mask = torch.zeros(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    for row0 in range(0, S, 256):
        n = min(256, S - row0)
        dsa.dsa_topk(sc[:, row0:row0 + n].contiguous(), None, B, S, K, row0, n, idx, mask)
    torch.cuda.synchronize()
    want = ref.topk(vals.double().numpy(), None, np.arange(S), K, S)
    assert np.array_equal(idx.cpu().numpy(), want)
    bits, cls = dsa.mask_views(mask, B, S)
    wb, wc = _mask_ref(want, S)
    assert np.array_equal(bits.cpu().numpy(), wb)
    assert np.array_equal(cls.cpu().numpy(), wc)


@pytest.mark.parametrize("segments", [None, (40, 200)])
def test_topk_vs_oracle_scores(segments):
    """End to end selection against the oracle's own scores and sets."""
    cfg = _cfg(S=600, K=128, segments=segments)
    x, d = _make(cfg)
    S, B, K = cfg.S, cfg.B, cfg.K
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, cfg.Dqk, cfg.Dv)
    path.select(d["q_idx"], d["k_idx"], d["w"], _seg_dev(x))
    torch.cuda.synchronize()
    rows = np.arange(S)
    rs = ref.index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), _seg_np(x), rows)
    ri = ref.topk(rs, _seg_np(x), rows, K, S)
    dec = compare_topk_rows(rs, f64(path.scores), path.idx.cpu().numpy(), ri, _seg_np(x), rows, S, K)
    assert len(dec) >= 0.9 * B * S


def _long_rows(B, n, S, row0, dtype, seed):
    """Scores of n slab rows with the structures the selection must handle:
    value ties, signed zeros, far outliers (outside a sampled value range),
    a single repeated value with a few larger ones, and constant rows."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn((B, n, S), generator=g)
    for r in range(n):
        kind = (row0 + r) % 5
        if kind == 0:
            v[:, r] = torch.round(v[:, r] * 64) / 64
        elif kind == 1:
            v[:, r][torch.rand((B, S), generator=g) < 0.05] = -0.0
            v[:, r][torch.rand((B, S), generator=g) < 0.05] = 0.0
        elif kind == 2:
            v[:, r] = 0.5
            pos = torch.randint(0, row0 + r + 1, (B, 12), generator=g)
            v[:, r].scatter_(1, pos, 100.0)
        elif kind == 3:
            pos = torch.randint(0, row0 + r + 1, (B, 40), generator=g)
            v[:, r].scatter_(1, pos, torch.where(torch.rand((B, 40), generator=g) < 0.5, 1e30, -1e30))
        else:
            v[:, r] = -1.25
    return v.to(dtype)


@pytest.mark.parametrize("score_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("segments,K", [(None, 300), ((3000, 20000), 300), (None, 3500)])
def test_topk_long_rows(score_dtype, segments, K):
    """Rows on both sides of 4096 keys (scores in VGPRs / longer rows read
    once into a list of their largest keys, with the multi-pass selection
    behind it; K = 3500 is too large for the list, so long rows go straight to
    the multi-pass kernel), as slab calls of whole query tiles, with ties,
    signed zeros, outliers and constant rows: bit-exact index lists and mask
    rows."""
    B = 2
    # slabs across 4096 keys, at 16K / 32K / 64K, and the ragged end at S
    if score_dtype == torch.float32:
        S, slabs = 33000, [(3968, 256), (16256, 256), (32640, 256), (32896, 104)]
    else:
        S, slabs = 66000, [(3968, 256), (32640, 256), (65408, 256), (65920, 80)]
    seg = None if segments is None else inputs.segment_ids(B, S, segments[0], segments[1], seed=3)
    seg_dev = None if seg is None else torch.from_numpy(seg).to(DEV).contiguous()
    idx = torch.full((B, S, K), -7, dtype=torch.int32, device=DEV)
    mask = torch.zeros(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    bits, _ = dsa.mask_views(mask, B, S)
    for i, (row0, n) in enumerate(slabs):
        sc = _long_rows(B, n, S, row0, score_dtype, seed=100 + i)
        dsa.dsa_topk(sc.to(DEV).contiguous(), seg_dev, B, S, K, row0, n, idx, mask)
        torch.cuda.synchronize()
        want = ref.topk(sc.double().numpy(), seg, np.arange(row0, row0 + n), K, S)
        del sc
        got = idx[:, row0:row0 + n].cpu().numpy()
        assert np.array_equal(got, want), row0
        wb = ref.pack_bits(ref.selection_matrix(want, S)).view(np.int64)
        assert np.array_equal(bits[:, row0:row0 + n].cpu().numpy(), wb), row0


@pytest.mark.parametrize("score_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", ["shifted", "median"])
def test_topk_long_rows_threshold_at_or_below_zero(score_dtype, case):
    """Rows longer than 4096 keys whose K-th largest score is negative or
    zero, so the single-read kernel lists keys of both signs (for bf16 the
    entries then carry the signed order key): "shifted" scores N(0,1) - 3 with
    K = 300, "median" scores rounded to 1/16 with signed zeros and K = 2048,
    about half of a row just past 4096 keys, so ties and -0 / +0 sit at the
    threshold. Bit-exact index lists and mask rows."""
    B, S = 2, 8192
    K = 300 if case == "shifted" else 2048
    idx = torch.full((B, S, K), -7, dtype=torch.int32, device=DEV)
    mask = torch.zeros(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    bits, _ = dsa.mask_views(mask, B, S)
    for i, (row0, n) in enumerate([(4096, 256), (8064, 128)]):
        g = torch.Generator().manual_seed(500 + i)
        v = torch.randn((B, n, S), generator=g)
        if case == "shifted":
            v -= 3.0
        else:
            v = torch.round(v * 16) / 16
            v[torch.rand((B, n, S), generator=g) < 0.05] = -0.0
        sc = v.to(score_dtype)
        dsa.dsa_topk(sc.to(DEV).contiguous(), None, B, S, K, row0, n, idx, mask)
        torch.cuda.synchronize()
        want = ref.topk(sc.double().numpy(), None, np.arange(row0, row0 + n), K, S)
        got = idx[:, row0:row0 + n].cpu().numpy()
        assert np.array_equal(got, want), row0
        wb = ref.pack_bits(ref.selection_matrix(want, S)).view(np.int64)
        assert np.array_equal(bits[:, row0:row0 + n].cpu().numpy(), wb), row0


@pytest.mark.parametrize("score_dtype,S", [(torch.float32, 5003), (torch.bfloat16, 5005)])
def test_topk_long_rows_unaligned(score_dtype, S):
    """Rows longer than 4096 keys whose starts are not 16-byte aligned (a
    row of S scores is not a whole number of 16-byte blocks), so the
    single-read kernel's first and last stages hold positions outside the
    row: bit-exact index lists and mask rows against the oracle."""
    B, K = 2, 700
    idx = torch.full((B, S, K), -7, dtype=torch.int32, device=DEV)
    mask = torch.zeros(dsa.dsa_mask_bytes(B, S), dtype=torch.uint8, device=DEV)
    bits, _ = dsa.mask_views(mask, B, S)
    for i, (row0, n) in enumerate([(4096, 128), (4992, S - 4992)]):
        sc = _long_rows(B, n, S, row0, score_dtype, seed=700 + i)
        dsa.dsa_topk(sc.to(DEV).contiguous(), None, B, S, K, row0, n, idx, mask)
        torch.cuda.synchronize()
        want = ref.topk(sc.double().numpy(), None, np.arange(row0, row0 + n), K, S)
        got = idx[:, row0:row0 + n].cpu().numpy()
        assert np.array_equal(got, want), row0
        wb = ref.pack_bits(ref.selection_matrix(want, S)).view(np.int64)
        assert np.array_equal(bits[:, row0:row0 + n].cpu().numpy(), wb), row0


# --------------------------------------------------------------- attention
def _sets(cfg, x):
    return inputs.random_index_sets(cfg.B, cfg.S, cfg.K, _seg_np(x), seed=cfg.seed + 1)


@pytest.mark.parametrize("S,K,segments", [(333, 64, None), (333, 64, (40, 150)), (200, 256, None),
                                          (130, 1, None)])
def test_build_mask_and_attention_fwd_mfma(S, K, segments):
    cfg = _cfg(S=S, K=K, segments=segments)
    x, d = _make(cfg)
    B = cfg.B
    sets = _sets(cfg, x)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, cfg.Dqk, cfg.Dv)
    path.build_mask(torch.from_numpy(sets).to(DEV), _seg_dev(x))
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    torch.cuda.synchronize()
    bits, cls = dsa.mask_views(path.mask, B, S)
    wb, wc = _mask_ref(sets, S)
    assert np.array_equal(bits.cpu().numpy(), wb)
    assert np.array_equal(cls.cpu().numpy(), wc)
    O, L = ref.attention_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), sets, _seg_np(x), cfg.softmax_scale,
                             np.arange(S))
    check_close("O", f64(path.o), O, bf16=True)
    np.testing.assert_allclose(path.lse.cpu().numpy(), L, rtol=0, atol=1e-4)


@pytest.mark.parametrize("dtype,Dqk,Dv", [("fp32", 64, 64), ("bf16", 64, 64), ("bf16", 128, 96)])
def test_attention_fwd_plain(dtype, Dqk, Dv):
    cfg = _cfg(S=200, K=32, Dqk=Dqk, Dv=Dv, dtype=dtype, scaled=dtype == "bf16", segments=(30, 90))
    x, d = _make(cfg)
    B, S = cfg.B, cfg.S
    sets = _sets(cfg, x)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, cfg.K, cfg.H, Dqk, Dv, dtype=cfg.torch_dtype())
    path.build_mask(torch.from_numpy(sets).to(DEV), _seg_dev(x))
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    torch.cuda.synchronize()
    O, L = ref.attention_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), sets, _seg_np(x), cfg.softmax_scale,
                             np.arange(S))
    check_close("O", f64(path.o), O, bf16=dtype == "bf16")
    np.testing.assert_allclose(path.lse.cpu().numpy(), L, rtol=0, atol=1e-4)


def test_attention_negative_control():
    """A single flipped index per row in the oracle's sets must fail the check."""
    cfg = _cfg(S=256, K=16, H=2)
    x, d = _make(cfg)
    B, S = cfg.B, cfg.S
    sets = _sets(cfg, x)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, cfg.K, cfg.H, cfg.Dqk, cfg.Dv)
    path.build_mask(torch.from_numpy(sets).to(DEV), None)
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    torch.cuda.synchronize()
    bad = sets.copy()
    rows = np.arange(100, S)
    for b in range(B):
        for t in rows:
            kept = bad[b, t][bad[b, t] >= 0]
            free = np.setdiff1d(np.arange(t + 1), kept)
            bad[b, t, 0] = free[0]
            bad[b, t] = np.sort(bad[b, t])
    O_bad, _ = ref.attention_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), bad[:, rows], None,
                                 cfg.softmax_scale, rows)
    with pytest.raises(AssertionError):
        check_close("O", f64(path.o)[:, rows], O_bad, bf16=True)


@pytest.mark.parametrize("S,K,segments,dtype,dims", [
    (333, 64, None, "bf16", (192, 128)), (333, 48, (40, 150), "bf16", (192, 128)),
    (150, 256, None, "bf16", (192, 128)), (200, 32, (30, 90), "fp32", (64, 64)),
    (200, 32, None, "bf16", (64, 64))])
def test_attention_bwd(S, K, segments, dtype, dims):
    Dqk, Dv = dims
    cfg = _cfg(S=S, K=K, segments=segments, dtype=dtype, scaled=dtype == "bf16", Dqk=Dqk, Dv=Dv, H=2)
    x, d = _make(cfg)
    B = cfg.B
    sets = _sets(cfg, x)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, Dqk, Dv, dtype=cfg.torch_dtype(), backward=True)
    path.build_mask(torch.from_numpy(sets).to(DEV), _seg_dev(x))
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    path.backward(d["q"], d["k"], d["v"], d["dout"], cfg.softmax_scale)
    torch.cuda.synchronize()
    dq, dk, dv = ref.attention_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), sets,
                                   _seg_np(x), cfg.softmax_scale)
    bf = dtype == "bf16"
    check_close("dq", f64(path.dq), dq, bf16=bf, rel=2e-2)
    check_close("dk", f64(path.dk), dk, bf16=bf, rel=2e-2)
    check_close("dv", f64(path.dv), dv, bf16=bf, rel=2e-2)


@pytest.mark.parametrize("S,K,segments", [(777, 48, (10, 100)), (640, 2048, None)])
def test_attention_bwd_parts_on_poisoned_workspace(S, K, segments):
    """prep, dK/dV and dQ called one by one on a workspace full of 0xFF bytes
    (NaN as fp32 and bf16) give what the whole call gives, and match the
    oracle: dQ reads only the dS tiles dK/dV wrote (short segments leave many
    tiles EMPTY; K >= S makes every causal tile FULL)."""
    cfg = _cfg(S=S, K=K, segments=segments, dtype="bf16", scaled=True, Dqk=192, Dv=128, H=2)
    x, d = _make(cfg)
    B = cfg.B
    sets = _sets(cfg, x)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, 192, 128, dtype=cfg.torch_dtype(), backward=True)
    path.build_mask(torch.from_numpy(sets).to(DEV), _seg_dev(x))
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    path.backward(d["q"], d["k"], d["v"], d["dout"], cfg.softmax_scale)
    whole = [t.clone() for t in (path.dq, path.dk, path.dv)]
    ws = torch.full_like(path.ws, 0xFF)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in whole)
    dsa.dsa_sparse_attn_bwd_prep(path.o, d["dout"], path.lse, 192, ws)
    dsa.dsa_sparse_attn_bwd_dkdv(d["q"], d["k"], d["v"], d["dout"], path.lse, path.mask, cfg.softmax_scale,
                                 dk, dv, ws)
    dsa.dsa_sparse_attn_bwd_dq(d["q"], d["k"], d["v"], d["dout"], path.lse, path.mask, cfg.softmax_scale,
                               dq, ws)
    torch.cuda.synchronize()
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), whole):
        assert torch.equal(got, want), name
    rdq, rdk, rdv = ref.attention_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), sets,
                                      _seg_np(x), cfg.softmax_scale)
    check_close("dq", f64(dq), rdq, bf16=True, rel=2e-2)
    check_close("dk", f64(dk), rdk, bf16=True, rel=2e-2)
    check_close("dv", f64(dv), rdv, bf16=True, rel=2e-2)


def test_end_to_end_tiny_fp32():
    """The 128-token fp32 workload: indexer, top-k and forward against the oracle."""
    cfg = inputs.CONFIGS["c1"]
    x, d = _make(cfg)
    B, S, K = cfg.B, cfg.S, cfg.K
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, cfg.Dqk, cfg.Dv, dtype=torch.float32)
    path.step(d, cfg.softmax_scale)
    torch.cuda.synchronize()
    rows = np.arange(S)
    rs = ref.index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), None, rows)
    ri = ref.topk(rs, None, rows, K, S)
    dec = compare_topk_rows(rs, f64(path.scores), path.idx.cpu().numpy(), ri, None, rows, S, K)
    assert len(dec) >= 0.9 * S
    O, L = ref.attention_fwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), ri, None, cfg.softmax_scale, rows)
    rr = np.array([r for _, r in dec])
    check_close("O", f64(path.o)[:, rr], O[:, rr], bf16=False)
    np.testing.assert_allclose(path.lse.cpu().numpy()[:, :, rr], L[:, :, rr], rtol=0, atol=1e-5)
