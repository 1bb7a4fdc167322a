"""Helpers of the GPU parity tests: host copies, the decidability rule for
top-k rows, and tolerance checks. No method arithmetic lives here; the
expected values always come from ``oracle.dsa_oracle``."""
from __future__ import annotations

import numpy as np
import torch

from oracle import dsa_oracle as ref

# floating-point bars: max-abs 2e-2 (bf16) / 1e-5 (fp32). The relative bar
# (error / max|reference|) is added because the bf16 inputs are scaled by
# 1/sqrt(d), so outputs are ~1e-3 and 2e-2 alone could not tell a wrong
# mask from a right one.
BF16_ATOL = 2e-2
BF16_REL = 1e-2
BF16_STORE = 2.0 ** -8   # largest relative error of one rounding to bf16
FP32_ATOL = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def check_close(name, got, want, bf16: bool, rel=None):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: non-finite pattern differs"
    diff = np.abs(got[fin] - want[fin])
    err = diff.max(initial=0.0)
    scale = np.abs(want[fin]).max(initial=0.0)
    if bf16:
        r = BF16_REL if rel is None else rel
        # the absolute bar holds over and above each output's own final rounding
        # to bf16 (at most 2^-8 |x|), which alone exceeds 2e-2 once |x| > 5
        over = diff - BF16_STORE * np.abs(want[fin])
        assert over.max(initial=0.0) <= BF16_ATOL, \
            f"{name}: max-abs {err:.3e} beyond {BF16_ATOL} + bf16 rounding of the reference"
        assert err <= r * scale + 1e-5, f"{name}: max-abs {err:.3e} > {r} * max|ref| {scale:.3e}"
    else:
        tol = FP32_ATOL * max(1.0, scale)
        assert err <= tol, f"{name}: max-abs {err:.3e} > {tol:.3e}"
    return err, scale


def row_decision(ref_keys, gpu_keys, valid, K):
    """Decidability of one row's top-k (page gap rule, with the tie reading).

    Returns (decidable, k_n, k_n1, tau). ref_keys/gpu_keys are float64 arrays
    over all positions; only ``valid`` ones matter.
    """
    kv = ref_keys[valid]
    n = min(K, kv.size)
    amax = np.abs(kv).max(initial=0.0)
    if n == kv.size:
        return True, None, None, 0.0
    srt = np.sort(kv)[::-1]
    k_n, k_n1 = srt[n - 1], srt[n]
    tau = 1e-4 * max(abs(k_n), abs(k_n1)) + 1e-6 * amax
    if k_n == k_n1:
        near = valid & (np.abs(ref_keys - k_n) <= tau)
        return bool(np.all(gpu_keys[near] == ref_keys[near])), k_n, k_n1, tau
    gap = k_n - k_n1
    dec = gap / max(abs(k_n), abs(k_n1)) > 1e-4 and gap > 1e-6 * amax
    return dec, k_n, k_n1, tau


def check_undecidable_row(ref_keys, valid, sel, K, k_n, k_n1, tau):
    kept = sel[sel >= 0]
    n = min(K, int(valid.sum()))
    assert kept.size == n
    assert np.all(valid[kept])
    assert np.all(ref_keys[kept] >= k_n - tau)
    dropped = np.setdiff1d(np.nonzero(valid)[0], kept)
    assert np.all(ref_keys[dropped] <= k_n1 + tau)


def compare_topk_rows(ref_scores, gpu_scores, gpu_idx, ref_idx, seg, rows, S, K):
    """Exact index lists on decidable rows; the near-tie rule on the rest.
    Returns the list of decidable (b, r) pairs."""
    B = ref_scores.shape[0]
    decidable = []
    for b in range(B):
        seg_b = None if seg is None else seg[b]
        for r, t in enumerate(rows):
            valid = ref.valid_row(seg_b, S, int(t))
            dec, k_n, k_n1, tau = row_decision(ref_scores[b, r], gpu_scores[b, r], valid, K)
            if dec:
                assert np.array_equal(gpu_idx[b, r], ref_idx[b, r]), (b, int(t))
                decidable.append((b, r))
            else:
                check_undecidable_row(ref_scores[b, r], valid, gpu_idx[b, r], K, k_n, k_n1, tau)
    return decidable
