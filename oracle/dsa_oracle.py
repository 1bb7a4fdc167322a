"""Float64 CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The HIP library
never calls it, and it shares no code with the HIP library. It is written
from the definitions in the pages and is slow on purpose: each step is the
plain formula with numpy primitives (matmul, sort), and there is no blocking,
fusion or reordering beyond what that formula states.

Sources (page title · section):
  [P3]  "DeepSeek3.2: Onboard sparse attention" · Background. DSA adds two
        parts to MLA: an indexer, whose index score is a parametric
        query-key product, and a non-parametric top-k that picks, for each
        query, the keys and values it attends to.
  [P3n] same page · "What this PR does", item 1. The naive implementation
        takes the top-k indices as an index mask and adds it to the regular
        attention mask of dot-product attention. Training only.
  [P3c] same page · item 2. The 671B indexer config is 64 index heads of
        dim 128, top-k 2048.
  [P2f] "Support Ring Attention with DeepSeek DSA Sparse Indexer" · "Forward
        Flow". The index mask is [batch, S, S] and shared by all heads. It is
        combined with the causal condition (a query sees keys at or before
        its own position, the diagonal included), and the kept logits are the
        query-key products multiplied by a softmax scale.
  [P2b] same page · "Backward Flow". dQ = dP K, dK = dP^T Q and dV = P^T dO,
        each masked the same way.
  [P2t] same page · "Tests". The index mask is threaded with and without
        segment IDs.
  [P3r] "DeepSeek3.2: Onboard sparse attention" · "What this PR does",
        item 4. The original indexer runs on quantized fp8 inputs (the fp8
        indexer section at the end states the readings of that format).
  [P3o] same page · item 1, Indexer: partial RoPE on the indexer's q and k,
        concatenated layout (the RoPE section at the end states the readings).
  [P2l] "Support Ring Attention with DeepSeek DSA Sparse Indexer" · "Isolated
        Flax NNX Auxiliary Loss" and "Loss Harvesting & Objective Injection":
        an indexer loss is added to the training objective, and its gradient
        reaches the indexer's query and key projections.
  [P5t] "Implement QK attention head chunking for CSA [Deepseek v4]" · the
        review of calculate_csa_indexer_loss: the teacher is a float32 softmax
        of the attention scores, zeroed on invalid tokens and summed over
        heads; the teacher's inputs carry no gradient (the KL section at the
        end states the readings).

  [P4c] "Add Flash Attention Support to Deepseek v4" · Description: the V4
        layers CSA (compression ratio 4) and HCA (ratio 128) attend over
        compressed KV blocks with block-aligned masks (causal, sliding
        window); compressed KV is padded to a multiple of the kernel's block.
  [P5c] "Implement QK attention head chunking for CSA [Deepseek v4]" ·
        Description: CSA works on compressed blocks, and its indexer scores
        queries against them (the compressed-attention section at the end
        states the readings).

The indexer formula is not printed on the pages. It is the standard one of
the method: I[t,s] = sum_j w[t,j] * ReLU(q_idx[t,j,:] . k_idx[s,:]), with a
per-token, per-index-head weight w and one index key per token shared by all
index heads. The readings of what the pages leave open are:
  * valid(t) = { s <= t : seg[s] == seg[t] }. The causal condition includes
    the diagonal; without segment IDs there is one segment. Selection is
    segment-aware.
  * The selection takes n = min(K, |valid(t)|) keys. The order is: larger
    score first, then smaller s first among equal scores. -0 and +0 are equal.
  * Index lists are ascending and padded with -1 to K entries.
  * A row with no kept key has O = 0, LSE = -inf and zero gradients.
  * The selection key of a bf16 score buffer is the score rounded to bf16
    (round to nearest, ties to even).

Parity status: every function here is pinned by the tests in
``tests/test_oracle_pins.py``. The pins are brute force on tiny inputs,
library routines (torch float64 SDPA and autograd), closed forms,
invariants, and hand-computed fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# validity: causal (diagonal included) and same segment          [P2f], [P2t]
# ----------------------------------------------------------------------------
def valid_row(seg_b, S: int, t: int) -> np.ndarray:
    """Boolean [S]: True for keys s that query t may attend to.

    s <= t (causal with the diagonal, [P2f]) and, when segment IDs are given,
    seg[s] equal to seg[t] ([P2t]).
    """
    ok = np.zeros(S, dtype=bool)
    ok[: t + 1] = True
    if seg_b is not None:
        ok &= np.asarray(seg_b) == seg_b[t]
    return ok


# ----------------------------------------------------------------------------
# a1: indexer scores                                              [P3], [P3c]
# ----------------------------------------------------------------------------
def index_scores_row(q_t, w_t, k_b, valid) -> np.ndarray:
    """Scores of one query over all keys: [S] float64, -inf outside ``valid``.

    q_t [Hi, Di] (the query's index vectors), w_t [Hi], k_b [S, Di] (the batch
    row's index keys), valid bool [S].
    """
    prod = np.asarray(q_t, np.float64) @ np.asarray(k_b, np.float64).T   # [Hi, S]: head j . key s
    score = np.asarray(w_t, np.float64) @ np.maximum(prod, 0.0)          # sum_j w_j ReLU(.)
    out = np.full(score.shape, NEG_INF)
    out[valid] = score[valid]
    return out


def index_scores(q_idx, k_idx, w, seg, rows) -> np.ndarray:
    """Indexer scores for the given query rows, in float64.

    q_idx [B,S,Hi,Di], k_idx [B,S,Di], w [B,S,Hi] (any float dtype; used at
    their exact values). seg [B,S] int or None. rows: 1-D array of query
    positions t. Returns [B, len(rows), S] float64, where entry (b, r, s) is
    I[b, t=rows[r], s] for s in valid(t) and -inf elsewhere.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, S, Hi, Di = q_idx.shape
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, S), NEG_INF, dtype=np.float64)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            out[b, r] = index_scores_row(q_idx[b, t], w[b, t], k_idx[b], valid_row(seg_b, S, int(t)))
    return out


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits. Write x = m * 2**e with 0.5 <= |m| < 1.
    Then m * 2**8 rounded to the nearest integer, with ties to even, gives
    the kept significand. Values at and below bf16's smallest normal are not
    produced by this workload. Infinities and zeros pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])
    out[fin] = np.ldexp(np.rint(m * 256.0), e - 8)
    return out


# ----------------------------------------------------------------------------
# a2: top-k selection                                                   [P3]
# ----------------------------------------------------------------------------
def topk_row(keys, valid, K: int) -> np.ndarray:
    """Selected key positions of one query row, ascending.

    keys: float [S] selection keys (the scores); valid: bool [S].
    n = min(K, |valid|) keys are taken. A larger key comes first. Among
    equal keys the smaller position comes first.
    """
    cand = np.nonzero(valid)[0]
    n = min(int(K), cand.size)
    kv = np.asarray(keys, dtype=np.float64)[cand]
    order = np.lexsort((cand, -kv))     # primary: descending key; then ascending s
    return np.sort(cand[order[:n]])


def topk(scores, seg, rows, K: int, S: int) -> np.ndarray:
    """Top-k index lists [B, len(rows), K] int32, ascending, padded with -1.

    ``scores`` is [B, len(rows), S] (the selection keys of those rows).
    Validity is recomputed from causality and segments, so entries outside
    valid(t) are never read.
    """
    scores = np.asarray(scores)
    B = scores.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, K), -1, dtype=np.int32)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            sel = topk_row(scores[b, r], valid_row(seg_b, S, int(t)), K)
            out[b, r, : sel.size] = sel
    return out


# ----------------------------------------------------------------------------
# a2/a3: selection bitmask and tile classes                     [P2f], [P3n]
# ----------------------------------------------------------------------------
def selection_matrix(idx, S: int) -> np.ndarray:
    """Boolean [B, S, S]: M[b,t,s] is True when s is in row t's index list."""
    idx = np.asarray(idx)
    B, n_rows, _ = idx.shape
    M = np.zeros((B, n_rows, S), dtype=bool)
    for b in range(B):
        for t in range(n_rows):
            sel = idx[b, t]
            M[b, t, sel[sel >= 0]] = True
    return M


def pack_bits(M) -> np.ndarray:
    """Pack a boolean [B, S, S] matrix into u64 words [B, S, ceil(S/64)].

    Bit (s % 64) of word s // 64 is M[b, t, s].
    """
    M = np.asarray(M, dtype=bool)
    B, R, S = M.shape
    W = (S + 63) // 64
    out = np.zeros((B, R, W), dtype=np.uint64)
    for s in range(S):
        out[:, :, s // 64] |= M[:, :, s].astype(np.uint64) << np.uint64(s % 64)
    return out


def tile_classes(M, TQ: int, TK: int) -> np.ndarray:
    """Tile class [B, ceil(S/TQ), ceil(Sk/TK)] uint8 of a selection matrix
    M [B, S, Sk] (Sk = S for token keys, the entry count for compressed keys).

    0 = no selected pair in the tile, 2 = every in-range pair (t < S, s < Sk)
    selected, 1 = otherwise.
    """
    M = np.asarray(M, dtype=bool)
    B, S, Sk = M.shape
    nq, nk = (S + TQ - 1) // TQ, (Sk + TK - 1) // TK
    out = np.zeros((B, nq, nk), dtype=np.uint8)
    for b in range(B):
        for i in range(nq):
            for j in range(nk):
                blk = M[b, i * TQ:(i + 1) * TQ, j * TK:(j + 1) * TK]
                out[b, i, j] = 2 if blk.all() else (1 if blk.any() else 0)
    return out


# ----------------------------------------------------------------------------
# a4: sparse attention forward                      [P3n], [P2f]
# ----------------------------------------------------------------------------
def _kept(idx_row, seg_b, S: int, t: int) -> np.ndarray:
    """Keys kept for query t: its index list, intersected again with causal and
    segment validity (the index mask is added to the regular mask, [P3n])."""
    sel = np.asarray(idx_row)
    sel = sel[sel >= 0]
    ok = valid_row(seg_b, S, t)
    return np.unique(sel[ok[sel]])


def attention_fwd_row(q_t, k_sel, v_sel, scale: float):
    """Softmax attention of one query over its kept keys, all heads.

    q_t [H, Dqk]; k_sel [n, H, Dqk], v_sel [n, H, Dv] are the kept keys'
    rows (n >= 1). Returns O [H, Dv] and LSE [H] (natural log).
    """
    H = q_t.shape[0]
    O = np.zeros((H, v_sel.shape[-1]))
    L = np.zeros(H)
    for h in range(H):
        logit = scale * (k_sel[:, h] @ q_t[h])       # [n]
        m = logit.max()
        e = np.exp(logit - m)
        Z = e.sum()
        O[h] = (e / Z) @ v_sel[:, h]
        L[h] = m + np.log(Z)
    return O, L


def attention_fwd(q, k, v, idx, seg, scale: float, rows):
    """Masked softmax attention for the given query rows, in float64.

    q,k [B,S,H,Dqk], v [B,S,H,Dv]. idx [B, len(rows), K] holds the index
    lists of those rows. Returns O [B, len(rows), H, Dv] and LSE
    [B, H, len(rows)] (natural log). A row with no kept key gives O = 0 and
    LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, _ = q.shape
    Dv = v.shape[-1]
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, rows.size, H, Dv))
    L = np.full((B, H, rows.size), NEG_INF)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            ks = _kept(idx[b, r], seg_b, S, int(t))
            if ks.size == 0:
                continue
            O[b, r], L[b, :, r] = attention_fwd_row(q[b, t], k[b, ks], v[b, ks], scale)
    return O, L


# ----------------------------------------------------------------------------
# a5-a7: backward                                                  [P2b]
# ----------------------------------------------------------------------------
def attention_bwd_row(q_t, k_sel, v_sel, dout_t, scale: float):
    """One query row's terms of the backward, all heads.

    q_t [H, Dqk], dout_t [H, Dv]; k_sel [n, H, Dqk], v_sel [n, H, Dv] are the
    kept keys' rows. Returns dq_t [H, Dqk] and this row's contributions
    dk_sel [n, H, Dqk], dv_sel [n, H, Dv] to the kept keys' gradients:
      P = softmax over kept s of scale * q_t . k_s
      D = sum_e dO(t,e) O(t,e),  dP(s) = dO(t) . v(s),  dS = P * (dP - D)
      dq(t) = scale * sum_s dS k(s),  dk(s) += scale * dS q(t),  dv(s) += P dO(t)
    """
    H = q_t.shape[0]
    dq_t = np.zeros_like(q_t)
    dk_sel = np.zeros_like(k_sel)
    dv_sel = np.zeros_like(v_sel)
    for h in range(H):
        logit = scale * (k_sel[:, h] @ q_t[h])
        e = np.exp(logit - logit.max())
        P = e / e.sum()                                  # [n]
        O = P @ v_sel[:, h]                              # [Dv]
        D = dout_t[h] @ O
        dP = v_sel[:, h] @ dout_t[h]                     # [n]
        dS = P * (dP - D)
        dq_t[h] = scale * (dS @ k_sel[:, h])
        dk_sel[:, h] = scale * np.outer(dS, q_t[h])
        dv_sel[:, h] = np.outer(P, dout_t[h])
    return dq_t, dk_sel, dv_sel


def attention_bwd(q, k, v, dout, idx, seg, scale: float, rows=None):
    """Gradients of sum(O * dout) w.r.t. q, k, v, in float64.

    idx [B, S, K] holds every row's index list. With ``rows`` given, idx is
    [B, len(rows), K] for those rows, and only their terms are summed (a row
    sample of the same sums). Returns dq, dk, dv in the shapes of q, k, v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, H, _ = q.shape
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            t = int(t)
            ks = _kept(idx[b, r], seg_b, S, t)
            if ks.size == 0:
                continue
            dq[b, t], dk_sel, dv_sel = attention_bwd_row(q[b, t], k[b, ks], v[b, ks], dout[b, t], scale)
            dk[b, ks] += dk_sel
            dv[b, ks] += dv_sel
    return dq, dk, dv


def attention_bwd_rows(q, k, v, dout, idx_rows, seg, scale: float, rows):
    """dq for the given query rows only: [B, len(rows), H, Dqk].

    It is the same formula as ``attention_bwd``. dq(t) needs only row t's
    kept set, so a sample of rows can be checked at any size.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, H, Dqk = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, rows.size, H, Dqk))
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            ks = _kept(idx_rows[b, r], seg_b, S, int(t))
            if ks.size == 0:
                continue
            for h in range(H):
                logit = scale * (k[b, ks, h] @ q[b, t, h])
                e = np.exp(logit - logit.max())
                P = e / e.sum()
                O = P @ v[b, ks, h]
                D = dout[b, t, h] @ O
                dS = P * (v[b, ks, h] @ dout[b, t, h] - D)
                dq[b, r, h] = scale * (dS @ k[b, ks, h])
    return dq


def attention_bwd_keys(q, k, v, dout, idx, seg, scale: float, keys, heads):
    """dk, dv of the given (key s, head h) pairs only.

    idx [B, S, K] holds every row's index list, because the queries that
    keep key s can sit anywhere at or after s. Returns dk [B, n, Dqk] and
    dv [B, n, Dv], where n = len(keys) and pair i is (keys[i], heads[i]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, H, Dqk = q.shape
    Dv = v.shape[-1]
    keys = np.asarray(keys, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    dk = np.zeros((B, keys.size, Dqk))
    dv = np.zeros((B, keys.size, Dv))
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for i, (s, h) in enumerate(zip(keys, heads)):
            for t in range(int(s), S):
                ks = _kept(idx[b, t], seg_b, S, t)
                pos = np.searchsorted(ks, s)
                if pos >= ks.size or ks[pos] != s:
                    continue
                logit = scale * (k[b, ks, h] @ q[b, t, h])
                e = np.exp(logit - logit.max())
                P = e / e.sum()
                O = P @ v[b, ks, h]
                D = dout[b, t, h] @ O
                dS = P[pos] * (v[b, s, h] @ dout[b, t, h] - D)
                dk[b, i] += scale * dS * q[b, t, h]
                dv[b, i] += P[pos] * dout[b, t, h]
    return dk, dv


# ----------------------------------------------------------------------------
# next row: fp8 indexer                                                [P3r]
# ----------------------------------------------------------------------------
# [P3r] "DeepSeek3.2: Onboard sparse attention" · "What this PR does", item 4:
# the original torch reference runs its indexer through quantization and fp8
# kernels (activation quantization, an fp8 GEMM and an fp8 index kernel). The
# page gives no format. Readings taken here:
#   * OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7) and 3 mantissa
#     bits; no infinities; largest finite magnitude 448; smallest normal 2**-6;
#     subnormals are multiples of 2**-9.
#   * One float32 scale per quantized row: per (token, index head) for q_idx,
#     per token for k_idx. scale = amax / 448 in float32, the row is divided by
#     it in float32 and rounded to the nearest e4m3 value, ties to even. An
#     all-zero row gets scale 0 and zero codes.
#   * The scores are the indexer formula on the dequantized values
#     code * scale; w keeps its own precision.
FP8_MAX = 448.0


def fp8_e4m3_round(x) -> np.ndarray:
    """Round values to the nearest OCP E4M3 value, ties to even, float64 out.

    Normal range (|x| >= 2**-6): write |x| = m * 2**e with 0.5 <= m < 1; the
    format keeps 4 significant bits, so m * 2**4 is rounded to an integer
    (ties to even) and scaled back. Below 2**-6 the grid is uniform with step
    2**-9. Magnitudes that round past 448 are outside the format; the
    quantizer below never produces them, and they raise here.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros_like(a)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 512.0) / 512.0
    nrm = ~sub & (a > 0)
    m, e = np.frexp(a[nrm])
    out[nrm] = np.ldexp(np.rint(m * 16.0), e - 4)
    if np.any(out > FP8_MAX):
        raise ValueError("value outside the e4m3 range")
    return np.copysign(out, x)


def fp8_e4m3_encode(v) -> np.ndarray:
    """uint8 codes of values already on the E4M3 grid (bit layout s eeee mmm)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = (a < 2.0 ** -6) & (a > 0)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)           # exponent field 0
    nrm = a >= 2.0 ** -6
    m, e = np.frexp(a[nrm])                                         # a = m 2**e, m in [0.5, 1)
    frac = np.rint(m * 16.0).astype(np.int64) - 8                   # 3 mantissa bits
    code[nrm] = ((e - 1 + 7) << 3) | frac
    code |= np.signbit(v).astype(np.int64) << 7
    return code.astype(np.uint8)


def fp8_e4m3_decode(code) -> np.ndarray:
    """float64 values of uint8 E4M3 codes (the NaN codes 0x7f / 0xff excluded)."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(c >> 7, -mag, mag)


def quantize_fp8_rows(x):
    """Quantize the last axis of x to E4M3 with one float32 scale per row.

    Returns (codes uint8, same shape as x; scale float32, x.shape[:-1]). The
    arithmetic is float32, as the readings above state: amax, scale =
    amax / 448 and x / scale are each rounded to float32 before the final
    rounding to E4M3.
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x32 / safe[..., None]).astype(np.float32)
    y = np.where(scale[..., None] > 0, y, np.float32(0.0))
    codes = fp8_e4m3_encode(fp8_e4m3_round(y.astype(np.float64)))
    return codes, scale


def index_scores_fp8(q8, q_scale, k8, k_scale, w, seg, rows) -> np.ndarray:
    """Indexer scores of fp8 inputs for the given query rows, in float64.

    q8 [B,S,Hi,Di] and k8 [B,S,Di] are E4M3 codes, q_scale [B,S,Hi] and
    k_scale [B,S] their float32 scales, w [B,S,Hi]. The scores are the
    indexer formula on the dequantized values (index_scores above).
    """
    q = fp8_e4m3_decode(q8) * np.asarray(q_scale, np.float64)[..., None]
    k = fp8_e4m3_decode(k8) * np.asarray(k_scale, np.float64)[..., None]
    return index_scores(q, k, w, seg, rows)


def index_scores_fp8_bound(q8, q_scale, k8, k_scale, w, rows, rel: float) -> np.ndarray:
    """Elementwise error bound [B, len(rows), S] for a kernel that forms each
    head's dot product q8 . k8 with an absolute error of at most
    rel * Di * max_d |q8_d| * max_d |k8_d| (in code units), and everything
    after it in float32:
        bound = sum_j |w_j| q_scale_j k_scale * rel * Di * max|q8_j| * max|k8|
              + 1e-6 * sum_j |w_j q_scale_j k_scale| * |q8_j| . |k8|.
    The second term covers float32 rounding of the products and the head sum.
    """
    qv = np.abs(fp8_e4m3_decode(q8))                      # [B,S,Hi,Di]
    kv = np.abs(fp8_e4m3_decode(k8))                      # [B,S,Di]
    w = np.abs(np.asarray(w, np.float64))
    qs = np.asarray(q_scale, np.float64)
    ks = np.asarray(k_scale, np.float64)
    B, _, Hi, Di = qv.shape
    S = kv.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, rows.size, S))
    for b in range(B):
        kmax = kv[b].max(axis=-1) * ks[b]                 # [S]
        for r, t in enumerate(rows):
            wq = w[b, t] * qs[b, t]                       # [Hi]
            mq = qv[b, t].max(axis=-1)                    # [Hi]
            dot_abs = qv[b, t] @ kv[b].T                  # [Hi, S]
            out[b, r] = rel * Di * (wq * mq).sum() * kmax + 1e-6 * (wq @ dot_abs) * ks[b]
    return out


# ----------------------------------------------------------------------------
# next row: indexer RoPE (partial, concatenated layout)                 [P3o]
# ----------------------------------------------------------------------------
# [P3o] "DeepSeek3.2: Onboard sparse attention" · "What this PR does", item 1,
# Indexer: the indexer applies partial RoPE to its q and k, with the same
# YaRN frequencies as MLA, in the concatenated layout rather than the
# interleaved one. Readings taken here:
#   * "partial": the first rope_dim dims of every index head vector (q_idx per
#     head, k_idx) are rotated, the rest pass through;
#   * "concatenated": dim i pairs with dim i + rope_dim/2 (not 2i with 2i+1);
#   * the frequencies arrive as tables cos[p, i], sin[p, i] (p a position,
#     i < rope_dim/2), so the YaRN construction stays with the caller; the
#     position of token t is pos[b, t] (t itself when no positions are given);
#   * the rotated vectors are bf16, like the inputs. Each output element is
#     float32(float32(x_a c) - float32(x_b s)) or float32(float32(x_b c) +
#     float32(x_a s)) rounded to bf16 (nearest, ties to even): the products
#     and the sum are each rounded to float32, with no fused multiply-add.
def rope_rotate(x, cos_t, sin_t, pos, rope_dim: int) -> np.ndarray:
    """Partial concatenated-layout RoPE of x [B, S, ..., D] (bf16 values as
    float, or float32). cos_t, sin_t [P, rope_dim/2] float32; pos [B, S] int
    or None. Returns float64 values on the bf16 grid, same shape as x."""
    x32 = np.asarray(x, dtype=np.float32)
    B, S = x32.shape[:2]
    h = rope_dim // 2
    p = np.broadcast_to(np.arange(S), (B, S)) if pos is None else np.asarray(pos)
    c = np.asarray(cos_t, np.float32)[p]                  # [B, S, h]
    s = np.asarray(sin_t, np.float32)[p]
    extra = x32.ndim - 3                                  # head axes between S and D
    c = c.reshape(c.shape[:2] + (1,) * extra + (h,))
    s = s.reshape(s.shape[:2] + (1,) * extra + (h,))
    a, b = x32[..., :h], x32[..., h:rope_dim]
    ya = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    yb = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    out = x32.astype(np.float64).copy()
    out[..., :h] = ya.astype(np.float32)
    out[..., h:rope_dim] = yb.astype(np.float32)
    return bf16_round(out)


def index_scores_fp8_rows(q8_rows, q_scale_rows, k8, k_scale, w_rows, seg, rows) -> np.ndarray:
    """index_scores_fp8 for long sequences: the query side is given only for
    the requested rows (q8_rows [B, R, Hi, Di], q_scale_rows [B, R, Hi],
    w_rows [B, R, Hi], R = len(rows)); keys for every position."""
    q = fp8_e4m3_decode(q8_rows) * np.asarray(q_scale_rows, np.float64)[..., None]
    k = fp8_e4m3_decode(k8) * np.asarray(k_scale, np.float64)[..., None]
    w_rows = np.asarray(w_rows, np.float64)
    B, S = k.shape[:2]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, S), NEG_INF)
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            out[b, r] = index_scores_row(q[b, r], w_rows[b, r], k[b], valid_row(seg_b, S, int(t)))
    return out


def index_scores_fp8_bound_rows(q8_rows, q_scale_rows, k8, k_scale, w_rows, rel: float) -> np.ndarray:
    """index_scores_fp8_bound with the query side given only for the rows
    (same layout as index_scores_fp8_rows)."""
    R = np.asarray(q8_rows).shape[1]
    return index_scores_fp8_bound(q8_rows, q_scale_rows, k8, k_scale, w_rows, np.arange(R), rel)


# ----------------------------------------------------------------------------
# next row: the indexer's KL auxiliary loss and its gradient     [P2l], [P5t]
# ----------------------------------------------------------------------------
# [P2l] says the indexer loss joins the objective and trains the indexer's q/k
# projections; [P5t] prints the teacher: a float32 softmax of attention
# scores, masked to valid tokens, summed over heads, with stop-gradient
# inputs. The pages print neither the student nor the divergence. Readings:
#   * kept(t): the sorted kept keys of row t (its index list, intersected with
#     valid(t), as the attention uses it);
#   * teacher p_t(s) = sum_h P_h(t,s) / sum_s' sum_h P_h(t,s') over s in
#     kept(t), where P_h is head h's attention probability over kept(t) (the
#     forward's P). Each P_h sums to 1, so p_t is the mean over heads of P_h.
#     It carries no gradient;
#   * student q_t(s) = softmax over s in kept(t) of I[t,s] (the indexer score);
#   * loss = (1/N) sum_t KL(p_t || q_t) = (1/N) sum_t sum_s p log(p / q) with
#     0 log 0 = 0, over the N rows with a non-empty kept(t);
#   * gradient: dloss/dI[t,s] = (q_t(s) - p_t(s)) / N on kept pairs, 0 else;
#     through I = sum_j w_j ReLU(u_j), u_j = q_idx[t,j] . k_idx[s], with
#     ReLU'(0) = 0, it reaches q_idx, k_idx and w.
def _kept_keys(idx_row, seg_b, S: int, t: int) -> np.ndarray:
    """kept(t) ascending: the index list intersected with valid(t)."""
    sel = np.asarray(idx_row)
    sel = sel[(sel >= 0) & (sel < S)]
    ok = valid_row(seg_b, S, t)
    return np.unique(sel[ok[sel]])


def indexer_teacher(q, k, idx, seg, scale: float, rows) -> np.ndarray:
    """Teacher distribution of each row over its kept keys, [B, len(rows), K]:
    entry i is p_t at the i-th smallest kept key (i < |kept(t)|), 0 after.
    q, k [B, S, H, Dqk]; idx [B, len(rows), K]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, S, H, _ = q.shape
    K = np.asarray(idx).shape[-1]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, rows.size, K))
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            ks = _kept_keys(idx[b, r], seg_b, S, int(t))
            if ks.size == 0:
                continue
            acc = np.zeros(ks.size)
            for h in range(H):
                logit = scale * (k[b, ks, h] @ q[b, t, h])
                e = np.exp(logit - logit.max())
                acc += e / e.sum()                           # P_h over kept(t)
            out[b, r, : ks.size] = acc / acc.sum()
    return out


def indexer_kl(scores, teacher, idx, seg, rows, S: int, n_norm=None):
    """Student softmax, KL divergence and its gradient w.r.t. the scores.

    scores [B, len(rows), S] (the indexer scores of the rows), teacher as
    indexer_teacher returns it, idx [B, len(rows), K]. n_norm is N (default:
    the number of non-empty rows among `rows`). Returns
      row_kl [B, len(rows)]  KL(p_t || q_t) (0 for empty rows),
      loss                   sum of row_kl / N,
      dscores [B, len(rows), S]  (q - p) / N on kept pairs, 0 elsewhere.
    """
    scores = np.asarray(scores, dtype=np.float64)
    teacher = np.asarray(teacher, dtype=np.float64)
    B = scores.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    row_kl = np.zeros((B, rows.size))
    dscores = np.zeros((B, rows.size, S))
    kept_rows = []
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            ks = _kept_keys(idx[b, r], seg_b, S, int(t))
            if ks.size == 0:
                continue
            x = scores[b, r, ks]
            m = x.max()
            logq = x - m - np.log(np.exp(x - m).sum())
            p = teacher[b, r, : ks.size]
            pos = p > 0
            row_kl[b, r] = np.sum(p[pos] * (np.log(p[pos]) - logq[pos]))
            kept_rows.append((b, r, ks, np.exp(logq), p))
    N = len(kept_rows) if n_norm is None else int(n_norm)
    for b, r, ks, qd, p in kept_rows:
        dscores[b, r, ks] = (qd - p) / N
    loss = row_kl.sum() / N if N else 0.0
    return row_kl, loss, dscores


def indexer_bwd(q_idx, k_idx, w, dscores, seg, rows):
    """Gradients of sum_{t,s} dscores[t,s] * I[t,s] w.r.t. the indexer inputs,
    for the given query rows (dscores [B, len(rows), S]; entries outside
    valid(t) must be 0). Returns dq_idx [B, len(rows), Hi, Di],
    dk_idx [B, S, Di] (the rows' contributions) and dw [B, len(rows), Hi]:
      u_j = q_idx[t,j] . k_idx[s],  dw[t,j] += g ReLU(u_j),
      dq_idx[t,j] += g w[t,j] [u_j > 0] k_idx[s],
      dk_idx[s]   += sum_j g w[t,j] [u_j > 0] q_idx[t,j].
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dscores = np.asarray(dscores, dtype=np.float64)
    B, S, Hi, Di = q_idx.shape
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, rows.size, Hi, Di))
    dk = np.zeros((B, S, Di))
    dw = np.zeros((B, rows.size, Hi))
    for b in range(B):
        seg_b = None if seg is None else np.asarray(seg)[b]
        for r, t in enumerate(rows):
            vs = np.nonzero(valid_row(seg_b, S, int(t)))[0]
            g = dscores[b, r, vs]                            # [n]
            u = q_idx[b, t] @ k_idx[b, vs].T                 # [Hi, n]
            G = g[None, :] * w[b, t][:, None] * (u > 0)      # dI/du_j times g
            dw[b, r] = (np.maximum(u, 0.0) * g[None, :]).sum(axis=1)
            dq[b, r] = G @ k_idx[b, vs]
            dk[b, vs] += G.T @ q_idx[b, t]
    return dq, dk, dw


# ----------------------------------------------------------------------------
# next row: compressed sparse attention (DeepSeek-V4 CSA)          [P4c], [P5c]
# ----------------------------------------------------------------------------
# [P4c] says only that CSA compresses KV at ratio 4 and needs block-aligned
# causal (and sliding-window) masks; [P5c] that its indexer scores queries
# against the compressed blocks. Neither gives the compressor, the block-level
# causal rule or the window. Readings taken here:
#   * The compressed K, V and index keys are inputs (the compressor's
#     arithmetic is not given; like RoPE it is preparation before the path).
#     There are Sk = floor(S / ratio) entries; entry c stands for tokens
#     ratio*c .. ratio*c + ratio - 1, and tokens past ratio*Sk have none.
#   * Block causality: query t sees entry c when the entry's whole block lies
#     at or before t, i.e. ratio*c + ratio - 1 <= t. Rows t < ratio - 1 see
#     nothing (O = 0, LSE = -inf). With ratio 1 this is DSA's causal rule.
#   * Indexer, top-k and attention are DSA's formulas over the visible
#     entries. No segment IDs (the pages do not say how compression meets
#     packed documents) and no sliding window (its size and combination are
#     not given).
def csa_valid_row(Sk: int, ratio: int, t: int) -> np.ndarray:
    """Boolean [Sk]: entry c is visible to query t when ratio*c + ratio - 1 <= t."""
    c = np.arange(Sk)
    return ratio * c + (ratio - 1) <= t


def csa_index_scores(q_idx, k_idx_c, w, ratio: int, rows) -> np.ndarray:
    """Indexer scores over the compressed index keys for the given query rows.

    q_idx [B,S,Hi,Di], k_idx_c [B,Sk,Di], w [B,S,Hi]. Returns [B, len(rows), Sk]
    float64: I[b, t, c] for visible c, -inf elsewhere.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k_idx_c = np.asarray(k_idx_c, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, Sk = k_idx_c.shape[:2]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, Sk), NEG_INF, dtype=np.float64)
    for b in range(B):
        for r, t in enumerate(rows):
            out[b, r] = index_scores_row(q_idx[b, t], w[b, t], k_idx_c[b], csa_valid_row(Sk, ratio, int(t)))
    return out


def csa_topk(scores, ratio: int, rows, K: int, Sk: int) -> np.ndarray:
    """Top-k lists [B, len(rows), K] int32 over the visible entries of each
    row (ascending, padded with -1); ``scores`` is [B, len(rows), Sk]."""
    scores = np.asarray(scores)
    B = scores.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.full((B, rows.size, K), -1, dtype=np.int32)
    for b in range(B):
        for r, t in enumerate(rows):
            sel = topk_row(scores[b, r], csa_valid_row(Sk, ratio, int(t)), K)
            out[b, r, : sel.size] = sel
    return out


def csa_attention_fwd(q, k_c, v_c, idx, ratio: int, scale: float, rows):
    """Softmax attention of the given query rows over their kept compressed
    entries (index list intersected with visibility).

    q [B,S,H,Dqk], k_c [B,Sk,H,Dqk], v_c [B,Sk,H,Dv], idx [B, len(rows), K]
    (entries outside [0, Sk) name no entry and are dropped).
    Returns O [B, len(rows), H, Dv] and LSE [B, H, len(rows)]; a row with no
    kept entry has O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k_c = np.asarray(k_c, dtype=np.float64)
    v_c = np.asarray(v_c, dtype=np.float64)
    B, Sk, H, _ = k_c.shape
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, rows.size, H, v_c.shape[-1]))
    L = np.full((B, H, rows.size), NEG_INF)
    for b in range(B):
        for r, t in enumerate(rows):
            ks = _csa_kept(idx[b, r], Sk, ratio, int(t))   # entries that do not exist are not visible
            if ks.size == 0:
                continue
            O[b, r], L[b, :, r] = attention_fwd_row(q[b, t], k_c[b, ks], v_c[b, ks], scale)
    return O, L


def _csa_kept(idx_row, Sk: int, ratio: int, t: int) -> np.ndarray:
    """Entries kept for query t: its index list within [0, Sk), cut to the visible ones."""
    sel = np.asarray(idx_row)
    sel = sel[(sel >= 0) & (sel < Sk)]
    return np.unique(sel[csa_valid_row(Sk, ratio, t)[sel]])


def csa_attention_bwd(q, k_c, v_c, dout, idx, ratio: int, scale: float):
    """Gradients of sum(O * dout) w.r.t. q, k_c, v_c over every row, in float64:
    DSA's backward (same P, dS and sums) over each row's kept compressed entries.
    idx [B, S, K]. Returns dq [B,S,H,Dqk], dk_c [B,Sk,H,Dqk], dv_c [B,Sk,H,Dv]."""
    q = np.asarray(q, dtype=np.float64)
    k_c = np.asarray(k_c, dtype=np.float64)
    v_c = np.asarray(v_c, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S = q.shape[:2]
    Sk = k_c.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_c)
    dv = np.zeros_like(v_c)
    for b in range(B):
        for t in range(S):
            ks = _csa_kept(idx[b, t], Sk, ratio, t)
            if ks.size == 0:
                continue
            dq[b, t], dk_sel, dv_sel = attention_bwd_row(q[b, t], k_c[b, ks], v_c[b, ks], dout[b, t], scale)
            dk[b, ks] += dk_sel
            dv[b, ks] += dv_sel
    return dq, dk, dv
