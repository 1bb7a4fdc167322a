"""Parity of the indexer RoPE kernel with the oracle (bit-exact: the result
is a bf16 value, both sides form it from the same float32 steps), and of the
indexer on rotated inputs."""
import numpy as np
import pytest
import torch

from gpu_util import f64
from oracle import dsa_oracle as ref
from sparse_attention_06_amd import dsa, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def _tables(P, h, base=10000.0, factor=1.0):
    inv = base ** (-np.arange(h) / h) / factor
    ang = np.arange(P)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@pytest.mark.parametrize("shape,rope_dim", [((2, 333, 64, 128), 64), ((2, 333, 1, 128), 64),
                                            ((1, 200, 3, 64), 16), ((1, 77, 2, 128), 128)])
@pytest.mark.parametrize("with_pos", [False, True])
@pytest.mark.parametrize("inplace", [False, True])
def test_rope_bit_exact(shape, rope_dim, with_pos, inplace):
    B, S, nh, D = shape
    g = torch.Generator().manual_seed(S + rope_dim)
    x = torch.randn(shape, generator=g).to(torch.bfloat16)
    P = S + 17
    c, s = _tables(P, rope_dim // 2, factor=4.0)
    pos = torch.randint(0, P, (B, S), generator=g, dtype=torch.int32) if with_pos else None
    xd = x.to(DEV)
    out = xd if inplace else torch.full_like(xd, float("nan"))
    dsa.dsa_indexer_rope(xd, rope_dim, torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV),
                         None if pos is None else pos.to(DEV), out)
    torch.cuda.synchronize()
    want = ref.rope_rotate(x.float().numpy(), c, s, None if pos is None else pos.numpy(), rope_dim)
    np.testing.assert_array_equal(f64(out), want)


def test_indexer_on_rotated_inputs():
    cfg = inputs.CONFIGS["c2"].replace(B=2, S=333, segments=(40, 150))
    x = inputs.make_index_inputs(cfg, device="cpu")
    S = cfg.S
    c, s = _tables(S, 32)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    q = x["q_idx"].to(DEV).contiguous()
    k = x["k_idx"].to(DEV).contiguous()
    dsa.dsa_indexer_rope(q, 64, cd, sd)
    dsa.dsa_indexer_rope(k, 64, cd, sd)
    seg_d = x["seg"].to(DEV).contiguous()
    sc = torch.full((cfg.B, S, S), float("nan"), device=DEV)
    dsa.dsa_index_scores(q, k, x["w"].to(DEV), seg_d, 0, S, sc)
    torch.cuda.synchronize()
    qr = ref.rope_rotate(x["q_idx"].float().numpy(), c, s, None, 64)
    kr = ref.rope_rotate(x["k_idx"].float().numpy(), c, s, None, 64)
    want = ref.index_scores(qr, kr, f64(x["w"]), x["seg"].numpy(), np.arange(S))
    got = f64(sc)
    fin = np.isfinite(want)
    rowmax = np.abs(np.where(fin, want, 0)).max(axis=-1, keepdims=True)
    assert np.all(np.abs(np.where(fin, got - want, 0)) <= 1e-5 * rowmax + 1e-7)
