"""Parity of the fp8 (E4M3) indexer and its row quantizer with the float64
oracle, through the C ABI.

The quantizer is integer work on the codes: bit-exact against the oracle's
quantizer, scales included. The indexer's inputs are quantized on the host by
the oracle, and its scores are compared element by element with the oracle's
scores of the dequantized values, within the bound
``oracle.index_scores_fp8_bound``: each head's code dot product may be off by
REL * Di * max|q8| * max|k8| (the fp8 MFMA accumulates more coarsely than
float32; an in-bounds probe of one v_mfma_f32_32x32x64_f8f6f4 on random
full-range codes measured at most 2^-12.9 of the largest code product, and a
Di = 128 dot product is two of them), plus float32 rounding of the rest.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64
from oracle import dsa_oracle as ref
from sparse_attention_06_amd import dsa, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
# per-head dot-product error allowance: REL * Di * max|q8| * max|k8| is
# 2^-10 of the largest code product at Di = 128 (4x the two-MFMA model)
REL = 2.0 ** -17


def _quant_host(x: torch.Tensor):
    codes, scale = ref.quantize_fp8_rows(x.float().cpu().numpy())
    return torch.from_numpy(codes), torch.from_numpy(scale)


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_fp8_rows_bit_exact(D, dtype):
    g = torch.Generator().manual_seed(D)
    rows = 301
    x = torch.randn(rows, D, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 2)
    x[7] = 0.0                                    # all-zero row: scale 0, zero codes
    x[11, 5] = 1e-6                               # tiny values land on the subnormal grid
    x[13] = 2.0 ** -9                             # a constant row: every code is 448
    x = x.to(dtype)
    codes = torch.full((rows, D), 0x7F, dtype=torch.uint8, device=DEV)
    scale = torch.full((rows,), float("nan"), device=DEV)
    dsa.dsa_quant_fp8_rows(x.to(DEV), codes, scale)
    torch.cuda.synchronize()
    want_c, want_s = _quant_host(x)
    np.testing.assert_array_equal(scale.cpu().numpy(), want_s.numpy())
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c.numpy())


def _fp8_inputs(cfg):
    x = inputs.make_index_inputs(cfg, device="cpu")
    q8, qs = _quant_host(x["q_idx"])
    k8, ks = _quant_host(x["k_idx"])
    return x, q8, qs, k8, ks


def _check(got, want, bound):
    fin = np.isfinite(want)
    assert np.all(np.isfinite(got[fin]))
    err = np.abs(np.where(fin, got - want, 0))
    assert np.all(err <= np.where(fin, bound, 0)), float((err / np.maximum(bound, 1e-30)).max())
    return float((err[fin] / bound[fin]).max(initial=0.0))


@pytest.mark.parametrize("segments", [None, (40, 150)])
@pytest.mark.parametrize("score_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("HiDi", [(64, 128), (32, 128), (64, 64), (32, 64)])
def test_indexer_fp8_parity(segments, score_dtype, HiDi):
    Hi, Di = HiDi
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, Hi=Hi, Di=Di, segments=segments)
    x, q8, qs, k8, ks = _fp8_inputs(cfg)
    S = cfg.S
    seg_np = None if x["seg"] is None else x["seg"].numpy()
    seg_d = None if x["seg"] is None else x["seg"].to(DEV).contiguous()
    sc = torch.full((cfg.B, S, S), float("nan"), dtype=score_dtype, device=DEV)
    dsa.dsa_index_scores_fp8(q8.to(DEV), qs.to(DEV), k8.to(DEV), ks.to(DEV), x["w"].to(DEV), seg_d, 0, S, sc)
    torch.cuda.synchronize()
    rows = np.arange(S)
    w64 = f64(x["w"])
    want = ref.index_scores_fp8(q8.numpy(), qs.numpy(), k8.numpy(), ks.numpy(), w64, seg_np, rows)
    bound = ref.index_scores_fp8_bound(q8.numpy(), qs.numpy(), k8.numpy(), ks.numpy(), w64, rows, REL)
    got = f64(sc)
    if score_dtype == torch.bfloat16:
        # the bf16 store rounds the float32 score: half a bf16 step more
        bound = bound + np.abs(np.where(np.isfinite(want), want, 0)) * 2.0 ** -8
    ratio = _check(got, want, bound)
    print(f"fp8 indexer Hi={Hi} Di={Di} seg={segments} {score_dtype}: max err / bound {ratio:.3f}")


@pytest.mark.parametrize("key", ["c3", "c5"])
def test_indexer_fp8_full_length_sampled_rows(key):
    """S = 32768 (fp32 scores) and 131072 (bf16 scores), 64 x 128 index heads:
    slabs of rows at the start, middle and end of the sequence against the
    oracle (only those rows' q_idx are quantized and uploaded; every key is)."""
    cfg = inputs.CONFIGS[key]
    sdt = torch.bfloat16 if cfg.score_dtype == "bf16" else torch.float32
    x = inputs.make_index_inputs(cfg, device="cpu")
    S, Hi, Di = cfg.S, cfg.Hi, cfg.Di
    k8, ks = _quant_host(x["k_idx"])
    q8_d = torch.zeros((1, S, Hi, Di), dtype=torch.uint8, device=DEV)
    qs_d = torch.zeros((1, S, Hi), dtype=torch.float32, device=DEV)
    k8_d, ks_d, w_d = k8.to(DEV), ks.to(DEV), x["w"].to(DEV)
    slabs = (0, 13, S // 2 - 4, S - 4)
    nrows = 4
    got, q8s, qss = [], [], []
    for row0 in slabs:
        q8r, qsr = _quant_host(x["q_idx"][:, row0:row0 + nrows])
        q8s.append(q8r.numpy())
        qss.append(qsr.numpy())
        q8_d[:, row0:row0 + nrows] = q8r.to(DEV)
        qs_d[:, row0:row0 + nrows] = qsr.to(DEV)
        sc = torch.full((1, nrows, S), float("nan"), dtype=sdt, device=DEV)
        dsa.dsa_index_scores_fp8(q8_d, qs_d, k8_d, ks_d, w_d, None, row0, nrows, sc)
        torch.cuda.synchronize()
        got.append(f64(sc))
    rows = np.concatenate([np.arange(r, r + nrows) for r in slabs])
    q8h, qsh = np.concatenate(q8s, axis=1), np.concatenate(qss, axis=1)
    w_rows = f64(x["w"])[:, rows]
    want = ref.index_scores_fp8_rows(q8h, qsh, k8.numpy(), ks.numpy(), w_rows, None, rows)
    bound = ref.index_scores_fp8_bound_rows(q8h, qsh, k8.numpy(), ks.numpy(), w_rows, REL)
    if sdt == torch.bfloat16:
        bound = bound + np.abs(np.where(np.isfinite(want), want, 0)) * 2.0 ** -8
    worst = _check(np.concatenate(got, axis=1), want, bound)
    print(f"fp8 indexer S={S}: max err / bound {worst:.3f}")


@pytest.mark.parametrize("segments", [None, (40, 150)])
def test_fp8_selection_end_to_end(segments):
    """fp8 indexer, then the top-k on its scores, against the oracle's top-k on
    the oracle's fp8 scores: exact index lists on decidable rows, the near-tie
    rule on the rest, and the selection mask equal to the index lists."""
    from gpu_util import compare_topk_rows
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, K=64, segments=segments)
    x, q8, qs, k8, ks = _fp8_inputs(cfg)
    S, K = cfg.S, cfg.K
    seg_np = None if x["seg"] is None else x["seg"].numpy()
    seg_d = None if x["seg"] is None else x["seg"].to(DEV).contiguous()
    sc = torch.empty((cfg.B, S, S), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.B, S, K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_mask_bytes(cfg.B, S), dtype=torch.uint8, device=DEV)
    dsa.dsa_index_scores_fp8(q8.to(DEV), qs.to(DEV), k8.to(DEV), ks.to(DEV), x["w"].to(DEV), seg_d, 0, S, sc)
    dsa.dsa_topk(sc, seg_d, cfg.B, S, K, 0, S, idx, mask)
    torch.cuda.synchronize()
    rows = np.arange(S)
    rs = ref.index_scores_fp8(q8.numpy(), qs.numpy(), k8.numpy(), ks.numpy(), f64(x["w"]), seg_np, rows)
    ri = ref.topk(rs, seg_np, rows, K, S)
    gi = idx.cpu().numpy()
    dec = compare_topk_rows(rs, f64(sc), gi, ri, seg_np, rows, S, K)
    assert len(dec) >= 0.9 * cfg.B * S, len(dec)
    bits, _ = dsa.mask_views(mask, cfg.B, S)
    want_bits = ref.pack_bits(ref.selection_matrix(gi, S))
    np.testing.assert_array_equal(bits.cpu().numpy().view(np.uint64), want_bits)
    print(f"fp8 selection seg={segments}: {len(dec)} of {cfg.B * S} rows decidable and exact")


def test_path_select_fp8_matches_direct_calls():
    """DSAPath.select_fp8 (slabbed) gives the same index lists and mask as one
    direct fp8 indexer + top-k call on the whole sequence."""
    from sparse_attention_06_amd.pipeline import DSAPath
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, K=64)
    x, q8, qs, k8, ks = _fp8_inputs(cfg)
    d = [t.to(DEV) for t in (q8, qs, k8, ks, x["w"])]
    path = DSAPath(cfg.B, cfg.S, cfg.Hi, cfg.Di, cfg.K, cfg.H, cfg.Dqk, cfg.Dv)
    path.select_fp8(*d)
    sc = torch.empty((cfg.B, cfg.S, cfg.S), device=DEV)
    idx = torch.empty((cfg.B, cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    mask = torch.empty(dsa.dsa_mask_bytes(cfg.B, cfg.S), dtype=torch.uint8, device=DEV)
    dsa.dsa_index_scores_fp8(*d, None, 0, cfg.S, sc)
    dsa.dsa_topk(sc, None, cfg.B, cfg.S, cfg.K, 0, cfg.S, idx, mask)
    torch.cuda.synchronize()
    assert torch.equal(path.idx, idx)
    assert torch.equal(path.mask, mask)
