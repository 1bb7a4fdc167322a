"""dsa_sparse_attn_bwd_noalloc (the backward with the library's own scratch
array instead of a workspace) against dsa_sparse_attn_bwd with a caller
workspace: two calls in a row, the second on a smaller input, through the C ABI.
The allocation-free call takes the recompute route for dQ; the reference call
runs on a workspace with room for the dS handoff, so the two also cross-check
the routes. Both must match bit for bit, and the oracle within the bf16 bars."""
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


def _case(S, K, H, segments, dtype="bf16", dims=(192, 128), B=2):
    cfg = inputs.CONFIGS["c2"].replace(B=B, S=S, H=H, K=K, backward=True, segments=segments, dtype=dtype,
                                       scaled=dtype == "bf16", Dqk=dims[0], Dv=dims[1])
    x = inputs.make(cfg, device="cpu")
    d = {k: (None if v is None else v.to(DEV).contiguous()) for k, v in x.items()}
    seg_np = None if x["seg"] is None else x["seg"].numpy()
    sets = inputs.random_index_sets(B, S, K, seg_np, seed=cfg.seed + 1)
    path = DSAPath(B, S, cfg.Hi, cfg.Di, K, H, dims[0], dims[1], dtype=cfg.torch_dtype(), backward=True)
    path.build_mask(torch.from_numpy(sets).to(DEV), d["seg"])
    path.forward(d["q"], d["k"], d["v"], cfg.softmax_scale)
    return cfg, x, d, sets, seg_np, path


def _noalloc(path, d, scale):
    out = [torch.full_like(t, float("nan")) for t in (path.dq, path.dk, path.dv)]
    dsa.dsa_sparse_attn_bwd_noalloc(d["q"], d["k"], d["v"], path.o, d["dout"], path.lse, path.mask, scale, *out)
    return out


@pytest.mark.parametrize("dtype,dims", [("bf16", (192, 128)), ("fp32", (64, 64))])
def test_noalloc_matches_workspace_call_twice(dtype, dims):
    # the first call is the larger one, so the second reuses scratch that still
    # holds the first call's D and LSE past its own range
    for S, K, H, seg in ((1000, 256, 3, (64, 500)), (333, 48, 2, None)):
        cfg, x, d, sets, seg_np, path = _case(S, K, H, seg, dtype, dims)
        got = _noalloc(path, d, cfg.softmax_scale)
        path.backward(d["q"], d["k"], d["v"], d["dout"], cfg.softmax_scale)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, (path.dq, path.dk, path.dv)):
            assert torch.equal(g, w), (S, name)
        rdq, rdk, rdv = ref.attention_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), sets, seg_np,
                                          cfg.softmax_scale)
        for name, g, w in zip(("dq", "dk", "dv"), got, (rdq, rdk, rdv)):
            check_close(name, f64(g), w, bf16=dtype == "bf16", rel=2e-2)

