"""Pins of the float64 oracle to things other than itself (CPU only).

Each pin comes from the mathematics or from an independent routine:
  * hand-computed fixtures (tests/golden/*.json, each citing its page);
  * brute-force scalar loops (math.fsum / math.exp) on tiny inputs;
  * library routines: torch float64 scaled_dot_product_attention, logsumexp
    and autograd, numpy argmax, torch's float32->bfloat16 rounding;
  * closed forms and invariants: top-k >= |valid| gives dense causal
    attention, K = 1 gives the argmax key's value, constant v passes through,
    ReLU(x) + ReLU(-x) = |x|, linearity in w, the gradient sum rules;
  * a complete property check of the top-k rule (every kept key beats every
    dropped key, ties resolved by position).
The last block plants plausible mistakes in copies of the oracle and shows
that a pin catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as ref
from sparse_attention_06_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(x):
    table = {"ln3": math.log(3.0), "ln4": math.log(4.0), "0.75ln3": 0.75 * math.log(3.0)}
    return table[x] if isinstance(x, str) else float(x)


def _tiny(B=2, S=9, Hi=3, Di=5, H=2, Dqk=4, Dv=3, seed=0, seg=True):
    rng = np.random.default_rng(seed)
    d = dict(
        q_idx=rng.standard_normal((B, S, Hi, Di)),
        k_idx=rng.standard_normal((B, S, Di)),
        w=rng.standard_normal((B, S, Hi)),
        q=rng.standard_normal((B, S, H, Dqk)),
        k=rng.standard_normal((B, S, H, Dqk)),
        v=rng.standard_normal((B, S, H, Dv)),
        dout=rng.standard_normal((B, S, H, Dv)),
    )
    d["seg"] = np.array([[1] * 4 + [2] * (S - 4)] + [[5] * S] * (B - 1), dtype=np.int32) if seg else None
    return d


# ---------------------------------------------------------------- indexer pins
def test_indexer_hand_fixture():
    g = _load("indexer_hand.json")
    q = np.array(g["q_idx"], float)
    k = np.array(g["k_idx"], float)
    w = np.array(g["w"], float)
    rows = np.arange(g["S"])
    for seg, key in ((None, "expected"), (np.array(g["seg"]), "expected_seg")):
        got = ref.index_scores(q, k, w, seg, rows)
        exp = np.array([[[(-np.inf if x is None else x) for x in r] for r in b] for b in g[key]])
        np.testing.assert_array_equal(got, exp)


def _brute_scores(q_idx, k_idx, w, seg, b, t):
    B, S, Hi, Di = q_idx.shape
    out = []
    for s in range(S):
        ok = s <= t and (seg is None or seg[b][s] == seg[b][t])
        if not ok:
            out.append(-math.inf)
            continue
        terms = []
        for j in range(Hi):
            dot = math.fsum(q_idx[b, t, j, d] * k_idx[b, s, d] for d in range(Di))
            terms.append(w[b, t, j] * max(dot, 0.0))
        out.append(math.fsum(terms))
    return out


@pytest.mark.parametrize("seg", [False, True])
def test_indexer_brute_force(seg):
    d = _tiny(seg=seg)
    B, S = d["q_idx"].shape[:2]
    got = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], d["seg"], np.arange(S))
    for b in range(B):
        for t in range(S):
            np.testing.assert_allclose(got[b, t], _brute_scores(d["q_idx"], d["k_idx"], d["w"], d["seg"], b, t),
                                       rtol=1e-12, atol=1e-12)


def test_indexer_relu_and_linearity_invariants():
    d = _tiny(seg=False)
    S = d["q_idx"].shape[1]
    rows = np.arange(S)
    I_pos = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], None, rows)
    I_neg = ref.index_scores(-d["q_idx"], d["k_idx"], d["w"], None, rows)
    absdot = np.abs(np.einsum("btjd,bsd->btjs", d["q_idx"], d["k_idx"]))
    expect = np.einsum("btj,btjs->bts", d["w"], absdot)
    causal = np.tril(np.ones((S, S), bool))
    np.testing.assert_allclose((I_pos + I_neg)[:, causal], expect[:, causal], rtol=1e-12, atol=1e-12)
    I_scaled = ref.index_scores(d["q_idx"], d["k_idx"], -2.5 * d["w"], None, rows)
    np.testing.assert_allclose(I_scaled[:, causal], -2.5 * I_pos[:, causal], rtol=1e-12)
    # Hi = 1, w = 1 and non-negative inputs: the score is the plain product
    qn, kn = np.abs(d["q_idx"][:, :, :1]), np.abs(d["k_idx"])
    I1 = ref.index_scores(qn, kn, np.ones_like(d["w"][:, :, :1]), None, rows)
    np.testing.assert_allclose(I1[:, causal], np.einsum("btd,bsd->bts", qn[:, :, 0], kn)[:, causal], rtol=1e-12)


def test_indexer_head_chunking_is_exact_sum():
    # the score summed over two halves of the index heads equals the full sum
    d = _tiny(Hi=6, seg=True)
    S = d["q_idx"].shape[1]
    rows = np.arange(S)
    full = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], d["seg"], rows)
    a = ref.index_scores(d["q_idx"][:, :, :3], d["k_idx"], d["w"][:, :, :3], d["seg"], rows)
    b = ref.index_scores(d["q_idx"][:, :, 3:], d["k_idx"], d["w"][:, :, 3:], d["seg"], rows)
    fin = np.isfinite(full)
    np.testing.assert_allclose(full[fin], (a + b)[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(fin, np.isfinite(a))


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(3)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 0.07,
                          rng.standard_normal(2000).astype(np.float32) * 1e3,
                          np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], np.float32)])
    # exact halfway cases between neighbouring bf16 values
    base = np.array([1.0, 1.0078125, 3.0, -5.0], np.float32).view(np.uint32)
    halves = (base + np.uint32(0x8000)).view(np.float32)
    x32 = np.concatenate([x32, halves])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = ref.bf16_round(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------- top-k pins
def test_topk_tie_fixture():
    g = _load("topk_ties.json")
    for c in g["cases"]:
        keys = np.array(c["keys"], float)
        S = keys.size
        got = ref.topk(keys[None, None, :], None, [c["t"]], c["K"], S)[0, 0]
        assert got.tolist() == c["expected"], c["why"]
    # the hand fixture's index lists
    gi = _load("indexer_hand.json")
    q, k, w = (np.array(gi[n], float) for n in ("q_idx", "k_idx", "w"))
    rows = np.arange(gi["S"])
    sc = ref.index_scores(q, k, w, None, rows)
    for kk in (1, 2):
        got = ref.topk(sc, None, rows, kk, gi["S"])
        assert got.tolist() == gi["topk"][f"K={kk}"]
    seg = np.array(gi["seg"])
    sc = ref.index_scores(q, k, w, seg, rows)
    assert ref.topk(sc, seg, rows, 2, gi["S"]).tolist() == gi["topk_seg"]["K=2"]


def _check_topk_properties(keys, valid, K, sel):
    """Complete specification of the selection rule for one row."""
    sel = np.asarray(sel)
    kept = sel[sel >= 0]
    cand = np.nonzero(valid)[0]
    n = min(K, cand.size)
    assert kept.size == n
    assert np.all(sel[n:] == -1)
    assert np.all(np.diff(kept) > 0)                       # ascending, distinct
    assert np.all(valid[kept])
    dropped = np.setdiff1d(cand, kept)
    for s in kept:                                         # every kept key beats every dropped key
        for u in dropped:
            assert keys[s] > keys[u] or (keys[s] == keys[u] and s < u)


def test_topk_complete_property_random_rows():
    rng = np.random.default_rng(7)
    for trial in range(300):
        S = int(rng.integers(1, 40))
        t = int(rng.integers(0, S))
        K = int(rng.integers(1, 45))
        # few distinct values so that ties are common; some signed zeros
        keys = rng.integers(-3, 4, size=S).astype(float) * 0.5
        keys[rng.random(S) < 0.1] = -0.0
        seg = rng.integers(0, 2, size=S) if trial % 2 else None
        valid = ref.valid_row(seg, S, t)
        sel = ref.topk(keys[None, None], None if seg is None else seg[None], [t], K, S)[0, 0]
        _check_topk_properties(keys, valid, K, sel)


def test_topk_special_cases():
    rng = np.random.default_rng(11)
    S = 50
    keys = rng.standard_normal(S)
    for t in (0, 7, 49):
        valid = ref.valid_row(None, S, t)
        # K >= |valid|: every valid key
        assert ref.topk_row(keys, valid, S + 3).tolist() == list(range(t + 1))
        # K = 1: numpy argmax (first occurrence on ties)
        assert ref.topk_row(keys, valid, 1).tolist() == [int(np.argmax(keys[: t + 1]))]
        # all keys equal: the n lowest positions
        assert ref.topk_row(np.zeros(S), valid, 5).tolist() == list(range(min(5, t + 1)))
    # distinct keys: the set equals the set of the n largest by a full sort
    for K in (1, 3, 17, 40):
        want = set(np.argsort(-keys[:45])[:K].tolist())
        assert set(ref.topk_row(keys, ref.valid_row(None, S, 44), K).tolist()) == want


# ----------------------------------------------------------- bitmask / tiles
def test_pack_bits_and_tile_classes_brute():
    rng = np.random.default_rng(5)
    B, S = 2, 131
    M = rng.random((B, S, S)) < 0.3
    M[:, :40, :30] = True               # a region of full tiles
    M[:, 100:, 64:] = False             # a region of empty tiles
    bits = ref.pack_bits(M)
    for b in range(B):
        for t in range(S):
            for s in range(S):
                assert bool((int(bits[b, t, s // 64]) >> (s % 64)) & 1) == M[b, t, s]
    TQ, TK = 16, 8
    cls = ref.tile_classes(M, TQ, TK)
    for b, i, j in itertools.product(range(B), range(cls.shape[1]), range(cls.shape[2])):
        vals = [M[b, t, s] for t in range(i * TQ, min(S, (i + 1) * TQ)) for s in range(j * TK, min(S, (j + 1) * TK))]
        want = 2 if all(vals) else (1 if any(vals) else 0)
        assert cls[b, i, j] == want
    idx = np.full((B, S, S), -1, np.int32)
    for b in range(B):
        for t in range(S):
            nz = np.nonzero(M[b, t])[0]
            idx[b, t, : nz.size] = nz
    assert np.array_equal(ref.selection_matrix(idx, S), M)
    # a rectangular selection (compressed keys): S rows, Sk keys
    Sk = 45
    Mr = rng.random((B, S, Sk)) < 0.4
    Mr[:, :32, :16] = True
    bits = ref.pack_bits(Mr)
    assert bits.shape == (B, S, 1)
    for b, t, s in itertools.product(range(B), range(S), range(Sk)):
        assert bool((int(bits[b, t, s // 64]) >> (s % 64)) & 1) == Mr[b, t, s]
    cls = ref.tile_classes(Mr, TQ, TK)
    assert cls.shape == (B, -(-S // TQ), -(-Sk // TK))
    for b, i, j in itertools.product(range(B), range(cls.shape[1]), range(cls.shape[2])):
        vals = [Mr[b, t, s] for t in range(i * TQ, min(S, (i + 1) * TQ)) for s in range(j * TK, min(Sk, (j + 1) * TK))]
        assert cls[b, i, j] == (2 if all(vals) else (1 if any(vals) else 0))


# --------------------------------------------------------- attention fwd pins
def test_attention_hand_fixture():
    g = _load("attention_hand.json")
    q = np.array([_num(x) for x in g["q"]]).reshape(1, 2, 1, 1)
    k = np.array([_num(x) for x in g["k"]]).reshape(1, 2, 1, 1)
    v = np.array([_num(x) for x in g["v"]]).reshape(1, 2, 1, 1)
    dout = np.array([_num(x) for x in g["dout"]]).reshape(1, 2, 1, 1)
    idx = np.array(g["idx"], np.int32)[None]
    O, L = ref.attention_fwd(q, k, v, idx, None, g["scale"], [0, 1])
    np.testing.assert_allclose(O[0, :, 0, 0], [_num(x) for x in g["O"]], rtol=1e-14)
    np.testing.assert_allclose(L[0, 0], [_num(x) for x in g["LSE"]], rtol=1e-14, atol=1e-15)
    dq, dk, dv = ref.attention_bwd(q, k, v, dout, idx, None, g["scale"])
    np.testing.assert_allclose(dq[0, :, 0, 0], [_num(x) for x in g["dq"]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dk[0, :, 0, 0], [_num(x) for x in g["dk"]], rtol=1e-14)
    np.testing.assert_allclose(dv[0, :, 0, 0], [_num(x) for x in g["dv"]], rtol=1e-14)


def _all_valid_idx(seg, B, S, K):
    idx = np.full((B, S, K), -1, np.int32)
    for b in range(B):
        for t in range(S):
            v = np.nonzero(ref.valid_row(None if seg is None else seg[b], S, t))[0][:K]
            idx[b, t, : v.size] = v
    return idx


@pytest.mark.parametrize("seg", [False, True])
def test_attention_topk_ge_S_is_dense_causal_sdpa(seg):
    d = _tiny(S=11, H=3, Dqk=6, Dv=5, seg=seg)
    q, k, v, sg = d["q"], d["k"], d["v"], d["seg"]
    B, S, H, Dqk = q.shape
    scale = 0.37
    # index lists from the oracle's own indexer + top-k with K >= S
    rows = np.arange(S)
    sc = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], sg, rows)
    idx = ref.topk(sc, sg, rows, S + 2, S)
    O, L = ref.attention_fwd(q, k, v, idx, sg, scale, rows)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    mask = torch.tril(torch.ones(S, S, dtype=torch.bool)).expand(B, 1, S, S).clone()
    if sg is not None:
        ts = torch.from_numpy(sg)
        mask &= (ts[:, None, :, None] == ts[:, None, None, :])
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(O, want.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    logits = (tq @ tk.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
    np.testing.assert_allclose(L, lse.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_k1_and_constant_v():
    d = _tiny(S=10, seg=False)
    q, k, v = d["q"], d["k"], d["v"]
    B, S, H, _ = q.shape
    rows = np.arange(S)
    sc = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], None, rows)
    idx = ref.topk(sc, None, rows, 1, S)
    O, L = ref.attention_fwd(q, k, v, idx, None, 0.5, rows)
    for b in range(B):
        for t in range(S):
            s = int(np.argmax(sc[b, t, : t + 1]))
            np.testing.assert_allclose(O[b, t], v[b, s], rtol=1e-14)
            np.testing.assert_allclose(L[b, :, t], 0.5 * np.einsum("hd,hd->h", q[b, t], k[b, s]), rtol=1e-12)
    vc = np.broadcast_to(np.arange(1, 4, dtype=float), v.shape).copy()
    idx = ref.topk(sc, None, rows, 4, S)
    O, _ = ref.attention_fwd(q, k, vc, idx, None, 0.5, rows)
    np.testing.assert_allclose(O, vc, rtol=1e-13)


def test_attention_brute_force_scalar():
    d = _tiny(S=9, seg=True)
    q, k, v, sg = d["q"], d["k"], d["v"], d["seg"]
    B, S, H, Dqk = q.shape
    rows = np.arange(S)
    sc = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], sg, rows)
    idx = ref.topk(sc, sg, rows, 3, S)
    O, L = ref.attention_fwd(q, k, v, idx, sg, 0.8, rows)
    for b, t, h in itertools.product(range(B), range(S), range(H)):
        ks = [int(s) for s in idx[b, t] if s >= 0]
        lg = [0.8 * math.fsum(q[b, t, h, i] * k[b, s, h, i] for i in range(Dqk)) for s in ks]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        Z = math.fsum(e)
        for c in range(v.shape[-1]):
            assert abs(math.fsum(e[i] / Z * v[b, s, h, c] for i, s in enumerate(ks)) - O[b, t, h, c]) < 1e-12
        assert abs(m + math.log(Z) - L[b, h, t]) < 1e-12


def test_attention_packing_invariance():
    # two documents packed in one row give the same outputs as run alone
    d = _tiny(B=1, S=12, seg=False)
    S1 = 5
    seg = np.array([[1] * S1 + [2] * (12 - S1)], np.int32)
    rows = np.arange(12)
    sc = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], seg, rows)
    idx = ref.topk(sc, seg, rows, 3, 12)
    O, L = ref.attention_fwd(d["q"], d["k"], d["v"], idx, seg, 0.6, rows)
    sl = slice(S1, 12)
    rows2 = np.arange(12 - S1)
    sc2 = ref.index_scores(d["q_idx"][:, sl], d["k_idx"][:, sl], d["w"][:, sl], None, rows2)
    idx2 = ref.topk(sc2, None, rows2, 3, 12 - S1)
    O2, L2 = ref.attention_fwd(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], idx2, None, 0.6, rows2)
    np.testing.assert_allclose(O[:, sl], O2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L[:, :, sl], L2, rtol=1e-13)


def test_attention_empty_row():
    d = _tiny(B=1, S=4, seg=False)
    idx = np.full((1, 4, 2), -1, np.int32)
    idx[0, 2, 0] = 3          # a future key: dropped by the causal condition
    O, L = ref.attention_fwd(d["q"], d["k"], d["v"], idx, None, 1.0, np.arange(4))
    assert np.all(O == 0) and np.all(L == -np.inf)
    dq, dk, dv = ref.attention_bwd(d["q"], d["k"], d["v"], d["dout"], idx, None, 1.0)
    assert not dq.any() and not dk.any() and not dv.any()


# --------------------------------------------------------- attention bwd pins
def _random_sets(B, S, K, seg, seed):
    return inputs.random_index_sets(B, S, K, seg, seed)


@pytest.mark.parametrize("seg", [False, True])
def test_attention_bwd_torch_autograd(seg):
    d = _tiny(S=10, H=2, Dqk=5, Dv=4, seg=seg)
    q, k, v, dout, sg = d["q"], d["k"], d["v"], d["dout"], d["seg"]
    B, S, H, _ = q.shape
    idx = _random_sets(B, S, 4, sg, seed=1)
    scale = 0.45
    dq, dk, dv = ref.attention_bwd(q, k, v, dout, idx, sg, scale)
    M = torch.from_numpy(ref.selection_matrix(idx, S))[:, None]              # [B,1,S,S]
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True) for x in (q, k, v))
    logits = (tq @ tk.transpose(-1, -2)) * scale
    P = torch.softmax(logits.masked_fill(~M, -math.inf), dim=-1)
    O = P @ tv
    (O * torch.from_numpy(dout).permute(0, 2, 1, 3)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


def test_attention_bwd_finite_differences():
    d = _tiny(B=1, S=6, H=1, Dqk=3, Dv=2, seg=False)
    q, k, v, dout = d["q"], d["k"], d["v"], d["dout"]
    S = q.shape[1]
    idx = _random_sets(1, S, 3, None, seed=2)
    scale = 0.9
    rows = np.arange(S)
    dq, dk, dv = ref.attention_bwd(q, k, v, dout, idx, None, scale)

    def f(q_, k_, v_):
        O, _ = ref.attention_fwd(q_, k_, v_, idx, None, scale, rows)
        return float(np.sum(O * dout))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for pos in itertools.product(*(range(n) for n in x.shape)):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args = {"q": q, "k": k, "v": v}
            num = (f(**{**{a + "_": b for a, b in args.items()}, name + "_": xp})
                   - f(**{**{a + "_": b for a, b in args.items()}, name + "_": xm})) / (2 * h)
            assert abs(num - g[pos]) < 1e-7, (name, pos, num, g[pos])


def test_attention_bwd_sum_rules_and_row_key_variants():
    d = _tiny(B=2, S=12, H=2, seg=True)
    q, k, v, dout, sg = d["q"], d["k"], d["v"], d["dout"], d["seg"]
    B, S, H, _ = q.shape
    idx = _random_sets(B, S, 5, sg, seed=3)
    dq, dk, dv = ref.attention_bwd(q, k, v, dout, idx, sg, 0.7)
    # sum_s dS(t, s) = 0 for every non-empty row, hence sum_s dk(s) = 0
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # sum_s P(t, s) = 1, hence sum_s dv(s) = sum_t dO(t)
    np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=1), rtol=1e-12, atol=1e-12)
    rows = np.array([0, 3, 11])
    np.testing.assert_allclose(ref.attention_bwd_rows(q, k, v, dout, idx[:, rows], sg, 0.7, rows), dq[:, rows],
                               rtol=1e-13, atol=1e-14)
    keys, heads = np.array([0, 4, 7, 11]), np.array([1, 0, 1, 0])
    dk_s, dv_s = ref.attention_bwd_keys(q, k, v, dout, idx, sg, 0.7, keys, heads)
    np.testing.assert_allclose(dk_s, dk[:, keys, heads], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv_s, dv[:, keys, heads], rtol=1e-13, atol=1e-14)


# -------------------------------------------------- planted mistakes are caught
def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Copies of oracle steps with one plausible mistake each; a pin must fail."""
    g = _load("indexer_hand.json")
    q, k, w = (np.array(g[n], float) for n in ("q_idx", "k_idx", "w"))
    expect = np.array([[[(-np.inf if x is None else x) for x in r] for r in b] for b in g["expected"]])

    def scores_no_relu(q_idx, k_idx, w_, rows):
        out = np.full((1, 3, 3), -np.inf)
        for t in rows:
            out[0, t, : t + 1] = (w_[0, t] @ (q_idx[0, t] @ k_idx[0].T))[: t + 1]
        return out

    def scores_w_inside(q_idx, k_idx, w_, rows):
        out = np.full((1, 3, 3), -np.inf)
        for t in rows:
            out[0, t, : t + 1] = np.maximum(w_[0, t][:, None] * (q_idx[0, t] @ k_idx[0].T), 0).sum(0)[: t + 1]
        return out

    def scores_strict_causal(q_idx, k_idx, w_, rows):
        out = ref.index_scores(q_idx, k_idx, w_, None, rows)
        for t in rows:
            out[0, t, t] = -np.inf
        return out

    for bad in (scores_no_relu, scores_w_inside, scores_strict_causal):
        assert not np.array_equal(bad(q, k, w, range(3)), expect), bad.__name__

    # wrong tie order (larger position first) breaks the tie fixture
    def topk_row_bad(keys, valid, K):
        cand = np.nonzero(valid)[0]
        order = np.lexsort((-cand, -np.asarray(keys)[cand]))
        return np.sort(cand[order[: min(K, cand.size)]])

    monkeypatch.setattr(ref, "topk_row", topk_row_bad)
    with pytest.raises(AssertionError):
        test_topk_tie_fixture()
    monkeypatch.undo()

    # a transposed softmax scale (dividing instead of multiplying) breaks SDPA parity
    orig = ref.attention_fwd

    def fwd_bad(q_, k_, v_, idx, seg, scale, rows):
        return orig(q_, k_, v_, idx, seg, 1.0 / scale, rows)

    monkeypatch.setattr(ref, "attention_fwd", fwd_bad)
    with pytest.raises(AssertionError):
        test_attention_topk_ge_S_is_dense_causal_sdpa(False)
    monkeypatch.undo()

    # a dropped D term in the backward (dS = P * dP) breaks the autograd pin
    def bwd_bad(q_, k_, v_, dout, idx, seg, scale):
        B, S, H, _ = q_.shape
        dq, dk, dv = np.zeros_like(q_), np.zeros_like(k_), np.zeros_like(v_)
        for b in range(B):
            for t in range(S):
                ks = ref._kept(idx[b, t], None if seg is None else seg[b], S, t)
                for h in range(H):
                    lg = scale * (k_[b, ks, h] @ q_[b, t, h])
                    P = np.exp(lg - lg.max())
                    P /= P.sum()
                    dS = P * (v_[b, ks, h] @ dout[b, t, h])
                    dq[b, t, h] = scale * (dS @ k_[b, ks, h])
                    dk[b, ks, h] += scale * np.outer(dS, q_[b, t, h])
                    dv[b, ks, h] += np.outer(P, dout[b, t, h])
        return dq, dk, dv

    monkeypatch.setattr(ref, "attention_bwd", bwd_bad)
    with pytest.raises(AssertionError):
        test_attention_bwd_torch_autograd(False)
    monkeypatch.undo()


# ------------------------------------------------------------- input recipe
def test_inputs_deterministic_and_distribution():
    cfg = inputs.CONFIGS["c2"].replace(B=1, S=256)
    a = inputs.make(cfg)
    b = inputs.make(cfg)
    for n in ("q", "k", "v", "q_idx", "k_idx", "w", "dout"):
        assert torch.equal(a[n], b[n]), n
        assert a[n].dtype == torch.bfloat16
    assert abs(a["q"].float().std().item() - 192 ** -0.5) < 0.01
    assert abs(a["w"].float().std().item() - 64 ** -0.5) < 0.01
    assert abs(a["dout"].float().std().item() - 1.0) < 0.05
    seg = inputs.segment_ids(4, 8192, 64, 4096, 0)
    for row in seg:
        assert row[0] == 1 and np.all(np.diff(row) >= 0) and np.all(np.diff(row) <= 1)
        _, counts = np.unique(row, return_counts=True)
        assert np.all(counts[:-1] >= 64) and np.all(counts[:-1] <= 4096)
    sets = inputs.random_index_sets(2, 50, 8, seg[:2, :50], 0)
    for b in range(2):
        for t in range(50):
            row = sets[b, t]
            kept = row[row >= 0]
            assert np.all(np.diff(kept) > 0) and np.all(kept <= t)
            assert np.all(seg[b, kept] == seg[b, t])


# ------------------------------------------------------------ fp8 indexer pins
def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)


def test_fp8_round_encode_decode_match_torch():
    # library pin: torch's float32 -> float8_e4m3fn conversion (round to nearest even)
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 60.0, rng.standard_normal(20000) * 0.01,
                        rng.uniform(-448.0, 448.0, 20000)]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    t = _torch_e4m3(x)
    np.testing.assert_array_equal(ref.fp8_e4m3_round(x), t.float().numpy())
    np.testing.assert_array_equal(ref.fp8_e4m3_encode(ref.fp8_e4m3_round(x)), t.view(torch.uint8).numpy())
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    dec = ref.fp8_e4m3_decode(codes)
    np.testing.assert_array_equal(dec, torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy())
    np.testing.assert_array_equal(ref.fp8_e4m3_encode(dec), codes)
    # hand cases: ties go to the even mantissa; the subnormal grid is 2**-9
    hand = {1.0625: 1.0, 1.1875: 1.25, 2.0 ** -10: 0.0, 3 * 2.0 ** -10: 2.0 ** -8, 0.3: 0.3125,
            447.0: 448.0, -240.0: -240.0, 2.0 ** -6: 2.0 ** -6}
    for a, b in hand.items():
        assert ref.fp8_e4m3_round(np.array([a]))[0] == b, a
    with pytest.raises(ValueError):
        ref.fp8_e4m3_round(np.array([470.0]))


def test_fp8_quantize_rows_properties():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((6, 5, 128)) * np.exp(rng.uniform(-3, 3, (6, 5, 1)))).astype(np.float32)
    x[2, 3] = 0.0                                       # an all-zero row
    codes, scale = ref.quantize_fp8_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32 and scale.shape == (6, 5)
    amax = np.abs(x).max(-1)
    np.testing.assert_array_equal(scale, (amax / np.float32(448.0)).astype(np.float32))
    assert scale[2, 3] == 0 and not codes[2, 3].any()
    dec = ref.fp8_e4m3_decode(codes)
    # the row's largest magnitude lands on (or next to) the format's largest value
    top = np.abs(dec).max(-1)
    assert np.all((top[scale > 0] >= 416.0) & (top[scale > 0] <= 448.0))
    # each code is the nearest e4m3 value to x / scale: half a step of relative error at most
    y = x / np.where(scale > 0, scale, 1)[..., None]
    err = np.abs(dec - y)
    step = np.where(np.abs(y) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(err <= step / 2 + 1e-9)
    # torch's conversion of the same float32 quotients gives the same codes
    yq = (x / np.where(scale > 0, scale, np.float32(1))[..., None]).astype(np.float32)
    yq[2, 3] = 0
    np.testing.assert_array_equal(codes, _torch_e4m3(yq).view(torch.uint8).numpy())


def test_fp8_indexer_brute_force_and_exact_values():
    rng = np.random.default_rng(13)
    B, S, Hi, Di = 2, 9, 3, 8
    q = rng.standard_normal((B, S, Hi, Di)).astype(np.float32)
    k = rng.standard_normal((B, S, Di)).astype(np.float32)
    w = rng.standard_normal((B, S, Hi))
    seg = np.array([[1] * 4 + [2] * 5, [3] * 9], dtype=np.int32)
    q8, qs = ref.quantize_fp8_rows(q)
    k8, ks = ref.quantize_fp8_rows(k)
    got = ref.index_scores_fp8(q8, qs, k8, ks, w, seg, np.arange(S))
    qd, kd = ref.fp8_e4m3_decode(q8), ref.fp8_e4m3_decode(k8)
    for b in range(B):
        for t in range(S):
            for s in range(S):
                if s > t or seg[b, s] != seg[b, t]:
                    assert got[b, t, s] == -np.inf
                    continue
                terms = []
                for j in range(Hi):
                    dot = math.fsum(float(qd[b, t, j, d]) * float(qs[b, t, j]) * float(kd[b, s, d]) * float(ks[b, s])
                                    for d in range(Di))
                    terms.append(w[b, t, j] * max(dot, 0.0))
                assert abs(got[b, t, s] - math.fsum(terms)) <= 1e-12 * (1 + abs(got[b, t, s]))
    # values on the e4m3 grid with unit scales: the pinned float64 indexer on the same numbers
    qe = rng.integers(-16, 17, (B, S, Hi, Di)).astype(np.float64) / 4
    ke = rng.integers(-16, 17, (B, S, Di)).astype(np.float64) / 8
    got = ref.index_scores_fp8(ref.fp8_e4m3_encode(qe), np.ones((B, S, Hi), np.float32),
                               ref.fp8_e4m3_encode(ke), np.ones((B, S), np.float32), w, None, np.arange(S))
    np.testing.assert_array_equal(got, ref.index_scores(qe, ke, w, None, np.arange(S)))
    # a positive key scale scales the key's scores (a power of two: exact in float32)
    ks2 = ks.copy()
    ks2[:, 4] *= np.float32(4.0)
    g1 = ref.index_scores_fp8(q8, qs, k8, ks, w, None, np.arange(S))
    g3 = ref.index_scores_fp8(q8, qs, k8, ks2, w, None, np.arange(S))
    np.testing.assert_allclose(g3[:, 4:, 4], 4.0 * g1[:, 4:, 4], rtol=1e-12)
    bound = ref.index_scores_fp8_bound(q8, qs, k8, ks, w, np.arange(S), rel=2.0 ** -12)
    assert bound.shape == (B, S, S) and np.all(bound > 0)
    assert not ref.index_scores_fp8_bound(q8, qs, k8, ks, 0 * w, np.arange(S), rel=2.0 ** -12).any()


def test_fp8_planted_mistakes_fail_a_pin(monkeypatch):
    # the other common e4m3 flavour (exponent bias 8, as in the FNUZ variant) breaks the torch pin
    def decode_bias8(code):
        c = np.asarray(code, dtype=np.int64)
        e, m = (c >> 3) & 15, c & 7
        mag = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
        return np.where(c >> 7, -mag, mag)

    monkeypatch.setattr(ref, "fp8_e4m3_decode", decode_bias8)
    with pytest.raises(AssertionError):
        test_fp8_round_encode_decode_match_torch()
    monkeypatch.undo()

    # rounding half away from zero instead of to even breaks the hand cases
    def round_away(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        m, e = np.frexp(a)
        out = np.where(a < 2.0 ** -6, np.floor(a * 512.0 + 0.5) / 512.0, np.ldexp(np.floor(m * 16.0 + 0.5), e - 4))
        return np.copysign(out, x)

    monkeypatch.setattr(ref, "fp8_e4m3_round", round_away)
    with pytest.raises(AssertionError):
        test_fp8_round_encode_decode_match_torch()
    monkeypatch.undo()

    # a dropped key scale breaks the brute-force pin
    orig = ref.index_scores_fp8

    def no_kscale(q8, qs, k8, ks, w, seg, rows):
        return orig(q8, qs, k8, np.ones_like(ks), w, seg, rows)

    monkeypatch.setattr(ref, "index_scores_fp8", no_kscale)
    with pytest.raises(AssertionError):
        test_fp8_indexer_brute_force_and_exact_values()
    monkeypatch.undo()


# ------------------------------------------------------------------ RoPE pins
def _rope_tables(P, h, base=10000.0):
    inv = base ** (-np.arange(h) / h)
    ang = np.arange(P)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32), ang


def _bf16(x):
    return ref.bf16_round(np.asarray(x, np.float64)).astype(np.float32)


def test_rope_identity_and_passthrough():
    rng = np.random.default_rng(21)
    x = _bf16(rng.standard_normal((2, 6, 3, 32)))
    h = 8
    out = ref.rope_rotate(x, np.ones((6, h), np.float32), np.zeros((6, h), np.float32), None, 2 * h)
    np.testing.assert_array_equal(out, x)                 # angle 0: identity, bit for bit
    c, s, _ = _rope_tables(6, h)
    out = ref.rope_rotate(x, c, s, None, 2 * h)
    np.testing.assert_array_equal(out[..., 2 * h:], x[..., 2 * h:])   # dims past rope_dim untouched
    np.testing.assert_array_equal(out[:, 0], x[:, 0])     # position 0 has angle 0


def test_rope_is_complex_rotation():
    # textbook form: (x_i + i x_{i+h}) * exp(i theta_i(p)); the oracle's float32
    # steps and bf16 output may differ from it by one bf16 step at most
    rng = np.random.default_rng(22)
    B, S, H, D, rd = 2, 50, 4, 128, 64
    h = rd // 2
    x = _bf16(rng.standard_normal((B, S, H, D)))
    c, s, ang = _rope_tables(S, h)
    got = ref.rope_rotate(x, c, s, None, rd)
    z = (x[..., :h].astype(np.float64) + 1j * x[..., h:rd]) * np.exp(1j * ang)[None, :, None, :]
    want = np.concatenate([z.real, z.imag], axis=-1)
    diff = np.abs(got[..., :rd] - want)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    assert np.all(diff <= ulp * 1.01 + 1e-12)
    assert np.mean(diff > ulp * 0.51) < 0.01             # almost everywhere the nearest bf16 value
    # rotation keeps the norm of every pair (up to bf16 rounding)
    n0 = np.hypot(x[..., :h], x[..., h:rd])
    n1 = np.hypot(got[..., :h], got[..., h:rd])
    assert np.allclose(n0, n1, rtol=2 ** -7, atol=1e-6)


def test_rope_relative_position_and_positions_argument():
    rng = np.random.default_rng(23)
    D, rd, S = 64, 64, 40
    h = rd // 2
    q = _bf16(rng.standard_normal((1, S, D)))
    k = _bf16(rng.standard_normal((1, S, D)))
    c, s, _ = _rope_tables(S, h)
    # all tokens share q's and k's vectors: <R(a)q, R(b)k> depends on a - b only
    qq = np.broadcast_to(q[:, :1], q.shape).copy()
    kk = np.broadcast_to(k[:, :1], k.shape).copy()
    rq = ref.rope_rotate(qq, c, s, None, rd)[0]
    rk = ref.rope_rotate(kk, c, s, None, rd)[0]
    d = {}
    for a in range(S):
        for b in range(a + 1):
            d.setdefault(a - b, []).append(float(rq[a] @ rk[b]))
    for v in d.values():
        assert max(v) - min(v) <= 0.05 * (1 + abs(np.mean(v)))
    # explicit positions select table rows
    pos = rng.integers(0, S, (1, S)).astype(np.int32)
    a = ref.rope_rotate(q, c, s, pos, rd)
    b = ref.rope_rotate(q, c[pos[0]], s[pos[0]], None, rd)   # row t reads table row pos[t] ... as position t
    np.testing.assert_array_equal(a, b)


def test_rope_planted_mistakes_fail_a_pin(monkeypatch):
    orig = ref.rope_rotate

    def interleaved(x, cos_t, sin_t, pos, rope_dim):
        x = np.asarray(x, np.float32)
        perm = np.arange(x.shape[-1])
        h = rope_dim // 2
        perm[:rope_dim] = np.concatenate([np.arange(0, rope_dim, 2), np.arange(1, rope_dim, 2)])
        y = orig(x[..., perm], cos_t, sin_t, pos, rope_dim)
        inv = np.argsort(perm)
        return y[..., inv]

    def wrong_sign(x, cos_t, sin_t, pos, rope_dim):
        return orig(x, cos_t, -np.asarray(sin_t), pos, rope_dim)

    for bad in (interleaved, wrong_sign):
        monkeypatch.setattr(ref, "rope_rotate", bad)
        with pytest.raises(AssertionError):
            test_rope_is_complex_rotation()
        monkeypatch.undo()


def test_fp8_row_restricted_helpers_match_full_functions():
    rng = np.random.default_rng(14)
    B, S, Hi, Di = 2, 11, 3, 16
    q8, qs = ref.quantize_fp8_rows(rng.standard_normal((B, S, Hi, Di)).astype(np.float32))
    k8, ks = ref.quantize_fp8_rows(rng.standard_normal((B, S, Di)).astype(np.float32))
    w = rng.standard_normal((B, S, Hi))
    seg = np.array([[1] * 5 + [2] * 6, [4] * 11], dtype=np.int32)
    rows = np.array([0, 4, 5, 10])
    full = ref.index_scores_fp8(q8, qs, k8, ks, w, seg, rows)
    part = ref.index_scores_fp8_rows(q8[:, rows], qs[:, rows], k8, ks, w[:, rows], seg, rows)
    np.testing.assert_array_equal(full, part)
    bf = ref.index_scores_fp8_bound(q8, qs, k8, ks, w, rows, 2.0 ** -17)
    bp = ref.index_scores_fp8_bound_rows(q8[:, rows], qs[:, rows], k8, ks, w[:, rows], 2.0 ** -17)
    np.testing.assert_array_equal(bf, bp)


# ------------------------------------------------ fp8 score error bound pins
# The fp8 indexer's parity tolerance is oracle.index_scores_fp8_bound. It is
# pinned here against an emulation of a coarse accumulator, written out
# independently of the bound: each head's dot product of codes is summed in
# 64-wide blocks, and every block's exact partial sum is rounded to a grid of
# 2^-13 of the largest code product inside that block, in the direction that
# moves the score furthest (towards sign(w_j)). That is the accumulation a
# K = 64 fp8 MFMA with ~13 fractional bits relative to its largest product
# would perform; everything after the dot product is exact here.
def _fp8_coarse_scores(q8, qs, k8, ks, w, rows, grid_rel=2.0 ** -13, block=64):
    qd, kd = ref.fp8_e4m3_decode(q8), ref.fp8_e4m3_decode(k8)   # code values
    B, S, Hi, Di = qd.shape
    out = np.full((B, len(rows), S), -np.inf)
    for b in range(B):
        for r, t in enumerate(rows):
            for s in range(t + 1):
                total = 0.0
                for j in range(Hi):
                    dot = 0.0
                    for d0 in range(0, Di, block):
                        prod = qd[b, t, j, d0:d0 + block] * kd[b, s, d0:d0 + block]
                        part = math.fsum(prod.tolist())
                        u = grid_rel * np.abs(prod).max()
                        if u > 0:
                            part = u * (math.ceil(part / u) if w[b, t, j] > 0 else math.floor(part / u))
                        dot += part
                    total += w[b, t, j] * float(qs[b, t, j]) * float(ks[b, s]) * max(dot, 0.0)
                out[b, r, s] = total
    return out


def _fp8_bound_case(seed=31, B=1, S=12, Hi=64, Di=128):
    """Codes whose largest |q8| and |k8| sit at the same dim of both 64-wide
    blocks (so a block's largest product is max|q8| * max|k8|), most head
    dot products positive, and key scales spread over 2^-4 .. 2^4."""
    rng = np.random.default_rng(seed)
    q = np.abs(rng.standard_normal((B, S, Hi, Di))).astype(np.float32) * 0.5
    k = np.abs(rng.standard_normal((B, S, Di))).astype(np.float32) * 0.5
    q[..., 3] = q[..., 67] = 4.0
    k[..., 3] = k[..., 67] = 4.0
    q *= np.where(rng.random((B, S, Hi, Di)) < 0.2, -1, 1).astype(np.float32)
    q8, qs = ref.quantize_fp8_rows(q)
    k8, ks = ref.quantize_fp8_rows(k)
    ks = (ks * np.exp2(rng.uniform(-4, 4, ks.shape))).astype(np.float32)
    w = rng.standard_normal((B, S, Hi))
    return q8, qs, k8, ks, w


def test_fp8_bound_covers_coarse_accumulation_and_is_tight():
    q8, qs, k8, ks, w = _fp8_bound_case()
    rows = np.arange(q8.shape[1])
    exact = ref.index_scores_fp8(q8, qs, k8, ks, w, None, rows)
    coarse = _fp8_coarse_scores(q8, qs, k8, ks, w, rows)
    fin = np.isfinite(exact)
    err = np.zeros_like(exact)
    err[fin] = np.abs(coarse[fin] - exact[fin])
    assert err.max() > 0
    # the bound the GPU tests use covers the emulated accumulator everywhere
    bound = ref.index_scores_fp8_bound(q8, qs, k8, ks, w, rows, rel=2.0 ** -17)
    assert np.all(err <= np.where(fin, bound, 0)), float((err / np.maximum(bound, 1e-300)).max())
    # and is not loose by an order of magnitude: an 8x tighter one is exceeded
    tight = ref.index_scores_fp8_bound(q8, qs, k8, ks, w, rows, rel=2.0 ** -20)
    assert np.any(err > np.where(fin, tight, np.inf))


def test_fp8_bound_planted_mistakes_fail_a_pin(monkeypatch):
    orig = ref.index_scores_fp8_bound

    def no_di(q8, q_scale, k8, k_scale, w, rows, rel):   # Di factor dropped
        return orig(q8, q_scale, k8, k_scale, w, rows, rel / np.asarray(q8).shape[-1])

    def no_kscale(q8, q_scale, k8, k_scale, w, rows, rel):   # k_scale dropped from the first term
        full = orig(q8, q_scale, k8, k_scale, w, rows, rel)
        small = orig(q8, q_scale, k8, k_scale, w, rows, 0.0)
        return small + (full - small) / np.asarray(k_scale, np.float64)[:, None, :]

    def head_max(q8, q_scale, k8, k_scale, w, rows, rel):    # max over heads instead of a sum
        Hi = np.asarray(q8).shape[2]
        per = [orig(q8[:, :, j:j + 1], q_scale[:, :, j:j + 1], k8, k_scale, w[:, :, j:j + 1], rows, rel)
               for j in range(Hi)]
        return np.max(per, axis=0)

    for bad in (no_di, no_kscale, head_max):
        monkeypatch.setattr(ref, "index_scores_fp8_bound", bad)
        with pytest.raises(AssertionError):
            test_fp8_bound_covers_coarse_accumulation_and_is_tight()
        monkeypatch.undo()


# ------------------------------------------------ indexer KL loss pins
# oracle.indexer_teacher / indexer_kl / indexer_bwd (the auxiliary loss of
# "Support Ring Attention with DeepSeek DSA Sparse Indexer", Loss Harvesting,
# with the teacher of "Implement QK attention head chunking for CSA
# [Deepseek v4]", review of calculate_csa_indexer_loss).
def _kl_case(seed=41, B=2, S=11, K=5, H=3, seg=True):
    d = _tiny(B=B, S=S, H=H, seed=seed, seg=seg)
    d["idx"] = inputs.random_index_sets(B, S, K, d["seg"], seed=seed)
    d["idx"][0, 6] = -1                                    # an empty row
    return d


def test_indexer_teacher_brute_force_and_attention_probabilities():
    d = _kl_case()
    B, S, H = d["q"].shape[:3]
    scale = 0.37
    rows = np.arange(S)
    p = ref.indexer_teacher(d["q"], d["k"], d["idx"], d["seg"], scale, rows)
    for b in range(B):
        for t in range(S):
            kept = sorted(set(int(s) for s in d["idx"][b, t] if s >= 0 and s <= t and
                              d["seg"][b, s] == d["seg"][b, t]))
            if not kept:
                assert not p[b, t].any()
                continue
            tot = [0.0] * len(kept)
            for h in range(H):
                lg = [scale * math.fsum(d["q"][b, t, h, e] * d["k"][b, s, h, e] for e in range(d["q"].shape[-1]))
                      for s in kept]
                m = max(lg)
                z = math.fsum(math.exp(x - m) for x in lg)
                for i, x in enumerate(lg):
                    tot[i] += math.exp(x - m) / z
            zz = math.fsum(tot)                                # summed over heads, then normalised
            for i in range(len(kept)):
                assert abs(p[b, t, i] - tot[i] / zz) <= 1e-13
            assert not p[b, t, len(kept):].any()
    # one head: the teacher is that head's attention probability exp(logit - LSE)
    q1, k1 = d["q"][:, :, :1], d["k"][:, :, :1]
    p1 = ref.indexer_teacher(q1, k1, d["idx"], d["seg"], scale, rows)
    _, L = ref.attention_fwd(q1, k1, d["v"][:, :, :1], d["idx"], d["seg"], scale, rows)
    b, t = 1, 9
    kept = ref._kept(d["idx"][b, t], d["seg"][b], S, t)
    want = np.exp(scale * (k1[b, kept, 0] @ q1[b, t, 0]) - L[b, 0, t])
    np.testing.assert_allclose(p1[b, t, : kept.size], want, rtol=1e-12)
    # invariant to the order of the heads
    perm = np.array([2, 0, 1])
    np.testing.assert_allclose(ref.indexer_teacher(d["q"][:, :, perm], d["k"][:, :, perm], d["idx"], d["seg"],
                                                   scale, rows), p, rtol=1e-13, atol=1e-15)


def test_indexer_kl_hand_fixture():
    # two kept keys, teacher (1/2, 1/2), scores (0, ln 3): student (1/4, 3/4),
    # KL = ln 2 / 2 + ln(2/3) / 2 = ln(4/3) / 2, gradient (q - p) / N = (-1/4, 1/4)
    # row 0 keeps only key 0 (KL 0), row 1 is empty, row 2 keeps keys 0 and 2
    S = 3
    idx = np.array([[[0, -1], [-1, -1], [0, 2]]], dtype=np.int32)
    scores = np.full((1, S, S), -np.inf)
    scores[0, 0, 0] = 0.0
    scores[0, 2, 0], scores[0, 2, 2] = 0.0, math.log(3.0)
    teacher = np.array([[[1.0, 0], [0, 0], [0.5, 0.5]]])
    row_kl, loss, ds = ref.indexer_kl(scores, teacher, idx, None, np.arange(S), S)
    assert row_kl[0, 0] == 0.0 and row_kl[0, 1] == 0.0
    assert abs(row_kl[0, 2] - 0.5 * math.log(4.0 / 3.0)) < 1e-15
    assert abs(loss - 0.25 * math.log(4.0 / 3.0)) < 1e-15            # N = 2 non-empty rows
    np.testing.assert_allclose(ds[0, 2], [-0.125, 0.0, 0.125], atol=1e-16)
    np.testing.assert_allclose(ds[0, 0], [0.0, 0.0, 0.0], atol=1e-16)  # one key: q = p = 1


def _dense_student_torch(scores, idx, seg, S):
    """Kept-key masks as a dense [B, S, S] bool array."""
    B = scores.shape[0]
    m = np.zeros((B, S, S), bool)
    for b in range(B):
        for t in range(S):
            kept = ref._kept(idx[b, t], None if seg is None else seg[b], S, t)
            m[b, t, kept] = True
    return m


def test_indexer_kl_matches_torch_kl_div_and_autograd():
    d = _kl_case()
    B, S = d["q"].shape[:2]
    rows = np.arange(S)
    scores = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], d["seg"], rows)
    teacher = ref.indexer_teacher(d["q"], d["k"], d["idx"], d["seg"], 0.5, rows)
    row_kl, loss, ds = ref.indexer_kl(scores, teacher, d["idx"], d["seg"], rows, S)
    mask = _dense_student_torch(scores, d["idx"], d["seg"], S)
    x = torch.tensor(np.where(mask, scores, 0.0), dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(mask)
    logq = torch.log_softmax(x.masked_fill(~tm, -math.inf), dim=-1)
    # teacher scattered to key positions
    pd = np.zeros((B, S, S))
    for b in range(B):
        for t in range(S):
            kept = np.nonzero(mask[b, t])[0]
            pd[b, t, kept] = teacher[b, t, : kept.size]
    P = torch.tensor(pd)
    nonempty = tm.any(dim=-1)
    per_row = torch.stack([torch.nn.functional.kl_div(logq[b, t][tm[b, t]], P[b, t][tm[b, t]], reduction="sum")
                           if nonempty[b, t] else torch.zeros((), dtype=torch.float64)
                           for b in range(B) for t in range(S)]).view(B, S)
    np.testing.assert_allclose(row_kl, per_row.detach().numpy(), rtol=1e-12, atol=1e-15)
    tl = per_row.sum() / nonempty.sum()
    assert abs(loss - tl.item()) < 1e-14
    tl.backward()
    np.testing.assert_allclose(ds, np.where(mask, x.grad.numpy(), 0.0), rtol=1e-10, atol=1e-15)
    assert np.all(row_kl >= -1e-15)
    # a student equal to the teacher (scores = log p + const) has zero loss and gradient
    same = np.where(mask, np.log(np.maximum(pd, 1e-300)) + 3.0, -np.inf)
    rk, l0, g0 = ref.indexer_kl(same, teacher, d["idx"], d["seg"], rows, S)
    assert abs(l0) < 1e-13 and np.abs(g0).max() < 1e-13


def test_indexer_bwd_matches_autograd_and_finite_differences():
    d = _kl_case(seed=43)
    B, S, Hi, Di = d["q_idx"].shape
    rows = np.arange(S)
    rng = np.random.default_rng(5)
    g = rng.standard_normal((B, S, S))
    for b in range(B):
        for t in range(S):
            g[b, t, ~ref.valid_row(d["seg"][b], S, t)] = 0.0
    dq, dk, dw = ref.indexer_bwd(d["q_idx"], d["k_idx"], d["w"], g, d["seg"], rows)
    # torch float64 autograd of sum(g * I) through a dense masked indexer
    q = torch.tensor(d["q_idx"], requires_grad=True)
    k = torch.tensor(d["k_idx"], requires_grad=True)
    w = torch.tensor(d["w"], requires_grad=True)
    u = torch.einsum("btjd,bsd->btjs", q, k)
    I = (w[..., None] * torch.relu(u)).sum(dim=2)                      # [B, S, S]
    (torch.tensor(g) * I).sum().backward()
    np.testing.assert_allclose(dq, q.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dk, k.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-11, atol=1e-13)
    # end to end: the loss as a function of the indexer inputs (teacher and
    # kept sets fixed), central finite differences against the chain rule
    teacher = ref.indexer_teacher(d["q"], d["k"], d["idx"], d["seg"], 0.5, rows)

    def loss_of(qi, ki, wi):
        sc = ref.index_scores(qi, ki, wi, d["seg"], rows)
        return ref.indexer_kl(sc, teacher, d["idx"], d["seg"], rows, S)[1]

    sc = ref.index_scores(d["q_idx"], d["k_idx"], d["w"], d["seg"], rows)
    _, _, ds = ref.indexer_kl(sc, teacher, d["idx"], d["seg"], rows, S)
    gq, gk, gw = ref.indexer_bwd(d["q_idx"], d["k_idx"], d["w"], ds, d["seg"], rows)
    h = 1e-6
    for arr, grad, pick in ((d["q_idx"], gq, (1, 7, 2, 3)), (d["k_idx"], gk, (0, 2, 4)), (d["w"], gw, (1, 8, 1)),
                            (d["q_idx"], gq, (0, 3, 0, 1)), (d["k_idx"], gk, (1, 5, 0))):
        xp, xm = arr.copy(), arr.copy()
        xp[pick] += h
        xm[pick] -= h
        args_p = [xp if arr is a else a for a in (d["q_idx"], d["k_idx"], d["w"])]
        args_m = [xm if arr is a else a for a in (d["q_idx"], d["k_idx"], d["w"])]
        fd = (loss_of(*args_p) - loss_of(*args_m)) / (2 * h)
        assert abs(fd - grad[pick]) <= 1e-7 * (1 + abs(fd)), (pick, fd, grad[pick])


def test_indexer_kl_planted_mistakes_fail_a_pin(monkeypatch):
    orig_t, orig_kl, orig_bwd = ref.indexer_teacher, ref.indexer_kl, ref.indexer_bwd

    def teacher_unnormalised(q, k, idx, seg, scale, rows):        # heads summed, not normalised
        return orig_t(q, k, idx, seg, scale, rows) * q.shape[2]

    def kl_reversed(scores, teacher, idx, seg, rows, S, n_norm=None):   # KL(q || p)
        scores = np.asarray(scores, np.float64)
        row_kl, loss, ds = orig_kl(scores, teacher, idx, seg, rows, S, n_norm)
        out = np.zeros_like(row_kl)
        for b in range(scores.shape[0]):
            for r, t in enumerate(rows):
                ks = ref._kept(idx[b, r], None if seg is None else seg[b], S, int(t))
                if ks.size:
                    x = scores[b, r, ks]
                    qd = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
                    p = np.maximum(teacher[b, r, : ks.size], 1e-300)
                    out[b, r] = np.sum(qd * (np.log(qd) - np.log(p)))
        return out, loss, ds

    def grad_sign(scores, teacher, idx, seg, rows, S, n_norm=None):     # (p - q) / N
        row_kl, loss, ds = orig_kl(scores, teacher, idx, seg, rows, S, n_norm)
        return row_kl, loss, -ds

    def bwd_no_w(q_idx, k_idx, w, dscores, seg, rows):               # w dropped from dq
        dq, dk, dw = orig_bwd(q_idx, k_idx, np.ones_like(w), dscores, seg, rows)
        return dq, orig_bwd(q_idx, k_idx, w, dscores, seg, rows)[1], dw

    def bwd_dw_linear(q_idx, k_idx, w, dscores, seg, rows):          # u instead of ReLU(u) in dw
        dq, dk, dw = orig_bwd(q_idx, k_idx, w, dscores, seg, rows)
        _, _, dwn = orig_bwd(-np.asarray(q_idx), k_idx, w, dscores, seg, rows)
        return dq, dk, dw - dwn

    for name, bad, test in (("indexer_teacher", teacher_unnormalised,
                             test_indexer_teacher_brute_force_and_attention_probabilities),
                            ("indexer_kl", kl_reversed, test_indexer_kl_matches_torch_kl_div_and_autograd),
                            ("indexer_kl", grad_sign, test_indexer_kl_matches_torch_kl_div_and_autograd),
                            ("indexer_bwd", bwd_no_w, test_indexer_bwd_matches_autograd_and_finite_differences),
                            ("indexer_bwd", bwd_dw_linear, test_indexer_bwd_matches_autograd_and_finite_differences)):
        monkeypatch.setattr(ref, name, bad)
        with pytest.raises(AssertionError):
            test()
        monkeypatch.undo()


# ---------------------------------------------------------------- compressed sparse attention (CSA)
def test_csa_visibility_brute_force():
    """csa_valid_row against the block-completeness reading, token by token:
    entry c is visible to t when every token of its block lies at or before t."""
    for ratio in (1, 2, 3, 4, 7):
        Sk = 40 // ratio
        for t in range(44):
            want = np.array([all(ratio * c + i <= t for i in range(ratio)) for c in range(Sk)], dtype=bool)
            assert np.array_equal(ref.csa_valid_row(Sk, ratio, t), want), (ratio, t)
    for t in range(30):  # ratio 1 is DSA's causal rule
        assert np.array_equal(ref.csa_valid_row(30, 1, t), ref.valid_row(None, 30, t))
    # the first complete block of ratio 4 ends at token 3
    assert not ref.csa_valid_row(10, 4, 2).any()
    assert np.array_equal(np.nonzero(ref.csa_valid_row(10, 4, 3))[0], [0])
    assert np.array_equal(np.nonzero(ref.csa_valid_row(10, 4, 8))[0], [0, 1])


def _on_token_axis(x_c, ratio, S):
    """Compressed entries placed at their blocks' last tokens ratio*c + ratio - 1 of
    a token axis of length S (zeros at every other position)."""
    x_c = np.asarray(x_c, dtype=np.float64)
    Sk = x_c.shape[1]
    out = np.zeros((x_c.shape[0], S) + x_c.shape[2:])
    out[:, ratio * np.arange(Sk) + ratio - 1] = x_c
    return out


def test_csa_equals_dsa_on_the_token_axis():
    """CSA over Sk compressed entries is DSA over the S token positions with
    entry c at p(c) = ratio*c + ratio - 1 and every other position excluded:
    the pinned DSA indexer, top-k and attention give the same scores, lists
    (mapped back to entries) and outputs."""
    rng = np.random.default_rng(5)
    B, S, ratio, Hi, Di, H, Dqk, Dv, K = 2, 39, 4, 3, 8, 2, 8, 6, 3
    Sk = S // ratio
    pos = ratio * np.arange(Sk) + ratio - 1
    q_idx = rng.standard_normal((B, S, Hi, Di))
    w = rng.standard_normal((B, S, Hi))
    k_idx_c = rng.standard_normal((B, Sk, Di))
    q = rng.standard_normal((B, S, H, Dqk))
    k_c = rng.standard_normal((B, Sk, H, Dqk))
    v_c = rng.standard_normal((B, Sk, H, Dv))
    scale = 0.4
    rows = np.arange(S)
    sc = ref.csa_index_scores(q_idx, k_idx_c, w, ratio, rows)
    idx_c = ref.csa_topk(sc, ratio, rows, K, Sk)
    O_c, L_c = ref.csa_attention_fwd(q, k_c, v_c, idx_c, ratio, scale, rows)
    k_tok = _on_token_axis(k_idx_c, ratio, S)
    on_grid = np.isin(np.arange(S), pos)
    idx_tok = np.full((B, S, K), -1, np.int32)
    for b in range(B):
        for t in range(S):
            valid_tok = ref.valid_row(None, S, t) & on_grid
            s_tok = ref.index_scores_row(q_idx[b, t], w[b, t], k_tok[b], valid_tok)
            np.testing.assert_allclose(sc[b, t], s_tok[pos], rtol=1e-12, atol=1e-12)
            sel_tok = ref.topk_row(s_tok, valid_tok, K)
            sel_c = idx_c[b, t][idx_c[b, t] >= 0]
            assert np.array_equal(pos[sel_c], sel_tok), (b, t)
            idx_tok[b, t, : sel_tok.size] = sel_tok
    O_t, L_t = ref.attention_fwd(q, _on_token_axis(k_c, ratio, S), _on_token_axis(v_c, ratio, S), idx_tok, None,
                                 scale, rows)
    np.testing.assert_allclose(O_c, O_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(L_c), np.isinf(L_t))
    fin = np.isfinite(L_t)
    np.testing.assert_allclose(L_c[fin], L_t[fin], rtol=1e-12, atol=1e-12)
    assert np.isinf(L_c[:, :, : ratio - 1]).all() and not O_c[:, : ratio - 1].any()  # rows before the first block


def test_csa_keep_all_is_block_causal_dense_attention():
    """Index lists naming every entry (future ones included) give torch float64
    SDPA over the compressed keys under the block-causal mask."""
    rng = np.random.default_rng(6)
    B, S, ratio, H, Dqk, Dv = 2, 29, 4, 3, 8, 5
    Sk = S // ratio
    q = rng.standard_normal((B, S, H, Dqk))
    k_c = rng.standard_normal((B, Sk, H, Dqk))
    v_c = rng.standard_normal((B, Sk, H, Dv))
    scale = 0.3
    rows = np.arange(S)
    idx = np.broadcast_to(np.arange(Sk, dtype=np.int32), (B, S, Sk)).copy()
    idx = np.concatenate([idx, np.full((B, S, 2), [Sk, -1], np.int32)], axis=-1)  # no entry Sk: dropped
    O, L = ref.csa_attention_fwd(q, k_c, v_c, idx, ratio, scale, rows)
    vis = np.array([[ratio * c + ratio - 1 <= t for c in range(Sk)] for t in range(S)])
    live = vis.any(axis=1)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)[:, :, live]
    tk = torch.from_numpy(k_c).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v_c).permute(0, 2, 1, 3)
    m = torch.from_numpy(vis[live])
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
    np.testing.assert_allclose(O[:, live], want.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    logits = torch.einsum("bhtd,bhsd->bhts", tq, tk) * scale
    lse = torch.logsumexp(logits.masked_fill(~m, -math.inf), dim=-1)
    np.testing.assert_allclose(L[:, :, live], lse.numpy(), rtol=1e-10, atol=1e-12)
    assert not O[:, ~live].any() and np.isinf(L[:, :, ~live]).all()


def test_csa_planted_mistakes_fail_a_pin(monkeypatch):
    orig_fwd = ref.csa_attention_fwd

    def from_block_start(Sk, ratio, t):      # sees a block from its first token
        return ratio * np.arange(Sk) <= t

    def one_token_late(Sk, ratio, t):        # needs one token past the block
        return ratio * np.arange(Sk) + ratio <= t

    def no_visibility_cut(q, k_c, v_c, idx, ratio, scale, rows):   # index list used as is
        saved = ref.csa_valid_row
        try:
            ref.csa_valid_row = lambda Sk, r, t: np.ones(Sk, dtype=bool)
            return orig_fwd(q, k_c, v_c, idx, ratio, scale, rows)
        finally:
            ref.csa_valid_row = saved

    for bad in (from_block_start, one_token_late):
        monkeypatch.setattr(ref, "csa_valid_row", bad)
        with pytest.raises(AssertionError):
            test_csa_visibility_brute_force()
        with pytest.raises(AssertionError):
            test_csa_keep_all_is_block_causal_dense_attention()
        monkeypatch.undo()
        monkeypatch.setattr(ref, "csa_valid_row", bad)
        with pytest.raises(AssertionError):
            test_csa_backward_equals_dsa_on_the_token_axis_and_autograd()
        monkeypatch.undo()
    monkeypatch.setattr(ref, "csa_attention_fwd", no_visibility_cut)
    with pytest.raises(AssertionError):
        test_csa_keep_all_is_block_causal_dense_attention()
    monkeypatch.undo()


def test_csa_backward_equals_dsa_on_the_token_axis_and_autograd():
    """CSA gradients: (1) the pinned DSA backward on the token axis (entry c at
    token ratio*c + ratio - 1, other positions never kept), gradients of the
    token positions mapped back; (2) with every entry listed, torch float64
    autograd through dense attention under the block-causal mask."""
    rng = np.random.default_rng(8)
    B, S, ratio, H, Dqk, Dv, K = 2, 27, 4, 2, 6, 5, 4
    Sk = S // ratio
    pos = ratio * np.arange(Sk) + ratio - 1
    q = rng.standard_normal((B, S, H, Dqk))
    k_c = rng.standard_normal((B, Sk, H, Dqk))
    v_c = rng.standard_normal((B, Sk, H, Dv))
    dout = rng.standard_normal((B, S, H, Dv))
    scale = 0.45
    tok = inputs.random_index_sets(B, S, K, None, seed=4)
    idx_c = np.where(tok >= 0, tok // ratio, -1).astype(np.int32)
    dq, dk, dv = ref.csa_attention_bwd(q, k_c, v_c, dout, idx_c, ratio, scale)
    idx_tok = np.full((B, S, K), -1, np.int32)
    for b in range(B):
        for t in range(S):
            kept = ref._csa_kept(idx_c[b, t], Sk, ratio, t)
            idx_tok[b, t, : kept.size] = pos[kept]
    dq_t, dk_t, dv_t = ref.attention_bwd(q, _on_token_axis(k_c, ratio, S), _on_token_axis(v_c, ratio, S), dout,
                                         idx_tok, None, scale)
    np.testing.assert_allclose(dq, dq_t, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, dk_t[:, pos], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, dv_t[:, pos], rtol=1e-12, atol=1e-12)
    off_grid = np.setdiff1d(np.arange(S), pos)
    assert not dk_t[:, off_grid].any() and not dv_t[:, off_grid].any()
    # keep-all against autograd
    idx_all = np.broadcast_to(np.arange(Sk, dtype=np.int32), (B, S, Sk)).copy()
    dq, dk, dv = ref.csa_attention_bwd(q, k_c, v_c, dout, idx_all, ratio, scale)
    vis = torch.from_numpy(np.array([[ratio * c + ratio - 1 <= t for c in range(Sk)] for t in range(S)]))
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k_c).requires_grad_()
    tv = torch.from_numpy(v_c).requires_grad_()
    logits = torch.einsum("bthd,bchd->bhtc", tq, tk) * scale
    logits = logits.masked_fill(~vis, -math.inf)
    p = torch.softmax(logits, dim=-1).nan_to_num(0.0)      # rows before the first block: no entry
    o = torch.einsum("bhtc,bchd->bthd", p, tv)
    (o * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
