"""Parity of the indexer KL auxiliary loss (teacher, student KL, gradients of
q_idx, k_idx and w) with the float64 oracle, through the C ABI.

Each call is checked on its own inputs: the teacher against
oracle.indexer_teacher on the same q, k and index sets; the KL call against
oracle.indexer_kl on the GPU's scores and teacher; the backward against
oracle.indexer_bwd on the GPU's score gradient. Tolerances: the teacher and
KL are float32 arithmetic (1e-5 relative to the row's largest value; the
score gradient (q - p)/N within 1e-5/N, q and p being probabilities); the
indexer gradients are bf16 outputs of bf16 MFMAs (G = g w rounded to bf16),
held to 2e-2 of the largest reference value, as the attention gradients.
"""
import numpy as np
import pytest
import torch

from gpu_util import check_close, f64
from oracle import dsa_oracle as ref
from sparse_attention_06_amd import dsa, inputs
from sparse_attention_06_amd.pipeline import DSAPath

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _case(S=333, K=64, H=3, segments=(40, 150), Dqk=192, Dv=128, B=2, empty_rows=False, own_sets=True):
    cfg = inputs.CONFIGS["c2"].replace(B=B, S=S, H=H, K=K, segments=segments, Dqk=Dqk, Dv=Dv, backward=False)
    x = inputs.make(cfg, device="cpu")
    d = {k: (None if v is None else v.to(DEV).contiguous()) for k, v in x.items()}
    seg = None if x["seg"] is None else x["seg"].numpy()
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, H, Dqk, Dv)
    path.select(d["q_idx"], d["k_idx"], d["w"], d["seg"])
    if empty_rows:
        # index lists with only future keys: the mask drops them, so the rows are empty
        idx = path.idx.cpu().numpy()
        for t in range(5, S - 1, 9):
            fut = np.arange(t + 1, min(S, t + 1 + K))
            idx[:, t] = -1
            idx[:, t, : fut.size] = fut
        path.idx.copy_(torch.from_numpy(idx))
        path.build_mask(path.idx, d["seg"])
        # dsa_indexer_kl expects dsa_topk's lists: kept keys ascending, then -1
        kept = np.full_like(idx, -1)
        for b in range(B):
            for t in range(S):
                ks = ref._kept(idx[b, t], None if seg is None else seg[b], S, t)
                kept[b, t, : ks.size] = ks
        path.idx.copy_(torch.from_numpy(kept))
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    torch.cuda.synchronize()
    return cfg, x, d, seg, path


@pytest.mark.parametrize("segments,Dqk,K,empty", [((40, 150), 192, 64, False), (None, 192, 64, True),
                                                  (None, 128, 2048, False), ((30, 90), 64, 32, False)])
def test_indexer_loss_parity(segments, Dqk, K, empty):
    cfg, x, d, seg, path = _case(segments=segments, Dqk=Dqk, K=K, empty_rows=empty)
    B, S = cfg.B, cfg.S
    scores_gpu = f64(path.scores).copy()
    idx = path.idx.cpu().numpy()
    path.indexer_loss(d, cfg.softmax_scale, inplace=True)
    torch.cuda.synchronize()
    rows = np.arange(S)
    # teacher on the same index sets
    want_t = ref.indexer_teacher(f64(x["q"]), f64(x["k"]), idx, seg, cfg.softmax_scale, rows)
    got_t = path.teacher.cpu().numpy().astype(np.float64)
    rowmax = np.abs(want_t).max(axis=-1, keepdims=True)
    assert np.all(np.abs(got_t - want_t) <= 2e-5 * rowmax + 1e-7), np.abs(got_t - want_t).max()
    nonempty = (idx[:, :, 0] >= 0)
    np.testing.assert_allclose(got_t.sum(axis=-1)[nonempty], 1.0, atol=1e-4)
    if empty:
        assert (~nonempty).any() and not got_t[~nonempty].any()
    # student KL on the GPU's scores and teacher
    row_kl, loss, ds = ref.indexer_kl(scores_gpu, got_t, idx, seg, rows, S)
    got_kl = path.row_kl.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_kl - row_kl) <= 1e-5 * (1 + np.abs(row_kl))), np.abs(got_kl - row_kl).max()
    lg = path.loss.cpu().numpy()
    assert lg[1] == nonempty.sum()
    assert abs(lg[0] - loss) <= 1e-5 * (1 + abs(loss))
    got_ds = f64(path.dscores)
    causal = np.tril(np.ones((S, S), bool))[None]
    # g = (q - p) / N with q, p in [0, 1] formed in float32: an absolute bar
    # (a relative one fails where q and p nearly cancel)
    err = np.where(causal, np.abs(got_ds - ds), 0)
    assert np.all(err <= 1e-5 / lg[1]), err.max() * lg[1]
    # indexer gradients on the GPU's score gradient
    g = np.where(causal, got_ds, 0.0)
    dq, dk, dw = ref.indexer_bwd(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), g, seg, rows)
    check_close("dq_idx", f64(path.dq_idx), dq, bf16=True, rel=2e-2)
    check_close("dk_idx", f64(path.dk_idx), dk, bf16=True, rel=2e-2)
    check_close("dw", f64(path.dw), dw, bf16=True, rel=2e-2)
    # end to end against the oracle's own teacher and scores (same index sets)
    rs = ref.index_scores(f64(x["q_idx"]), f64(x["k_idx"]), f64(x["w"]), seg, rows)
    _, loss_ref, _ = ref.indexer_kl(rs, want_t, idx, seg, rows, S)
    assert abs(lg[0] - loss_ref) <= 1e-4 * (1 + abs(loss_ref))


def test_indexer_loss_deterministic():
    cfg, x, d, seg, path = _case(S=1000, K=256, H=4, segments=(64, 500))
    scores = path.scores.clone()
    outs = []
    for _ in range(2):
        path.scores.copy_(scores)
        path.indexer_loss(d, cfg.softmax_scale, inplace=True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (path.teacher, path.row_kl, path.loss, path.dq_idx, path.dk_idx, path.dw)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_indexer_loss_fullsize_sampled():
    """The 2B training shape: teacher, KL and dq_idx/dw of sampled rows, and
    dk_idx of sampled keys (the oracle sums every query of the key's column)."""
    cfg = inputs.CONFIGS["c2"]
    x = inputs.make(cfg, device=DEV)
    B, S, K = cfg.B, cfg.S, cfg.K
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, cfg.H, cfg.Dqk, cfg.Dv)
    path.select(x["q_idx"], x["k_idx"], x["w"], None)
    path.forward(x["q"], x["k"], x["v"], cfg.softmax_scale)
    rng = np.random.default_rng(11)
    rows = np.unique(np.r_[0, 1, K - 1, K, S - 1, rng.integers(0, S, 24)])
    b = 5
    scores_rows = f64(path.scores[b, torch.from_numpy(rows).to(DEV)])
    idx_rows = path.idx[b, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    path.indexer_loss(x, cfg.softmax_scale, inplace=True)
    torch.cuda.synchronize()

    def g(name):
        return f64(x[name][b:b + 1])

    q, k = g("q"), g("k")
    want_t = ref.indexer_teacher(q, k, idx_rows[None], None, cfg.softmax_scale, rows)[0]
    got_t = path.teacher[b, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_t - want_t) <= 2e-5 * np.abs(want_t).max(axis=-1, keepdims=True) + 1e-7)
    N = float(path.loss[1].item())
    assert N == B * S
    row_kl, _, ds = ref.indexer_kl(scores_rows[None], got_t[None], idx_rows[None], None, rows, S, n_norm=N)
    got_kl = path.row_kl[b, torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_kl - row_kl[0]) <= 1e-5 * (1 + np.abs(row_kl[0])))
    got_ds = f64(path.dscores[b, torch.from_numpy(rows).to(DEV)])
    causal = np.arange(S)[None, :] <= rows[:, None]
    err = np.where(causal, np.abs(got_ds - ds[0]), 0)
    assert np.all(err <= 1e-5 / N), err.max() * N
    # dq_idx and dw of the sampled rows from their gradient rows
    qi, ki, wi = g("q_idx"), g("k_idx"), g("w")
    dq, _, dw = ref.indexer_bwd(qi, ki, wi, np.where(causal, got_ds, 0)[None], None, rows)
    check_close("dq_idx", f64(path.dq_idx[b, torch.from_numpy(rows).to(DEV)]), dq[0], bf16=True, rel=2e-2)
    check_close("dw", f64(path.dw[b, torch.from_numpy(rows).to(DEV)]), dw[0], bf16=True, rel=2e-2)
    # dk_idx of sampled keys: every query t >= s of the batch row contributes
    for s in (0, 1000, S - 2):
        col = f64(path.dscores[b, s:, s])                       # g(t, s) for t >= s
        u = np.einsum("tjd,d->tj", qi[0, s:], ki[0, s])          # [S - s, Hi]
        G = col[:, None] * wi[0, s:] * (u > 0)
        want = np.einsum("tj,tjd->d", G, qi[0, s:])
        got = f64(path.dk_idx[b, s])
        assert np.abs(got - want).max() <= 2e-2 * np.abs(want).max() + 1e-12, s
