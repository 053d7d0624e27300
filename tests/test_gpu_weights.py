"""The output weights of every row sum to one.

When every value row is the same vector c, softmax attention returns c for
every query row, whatever the scores: the weights are non-negative and sum to
one. The kernel multiplies V by bf16-rounded P and divides by the sum of
exactly those rounded values, so this holds up to fp32 accumulation rounding.
It holds on the longest rows too: the last-Q rows of a 128K triangle layer and
the last rows of a dense layer keep all 2048 key tiles, so any systematic drift
in a running sum over 4096 halves would show here. Peaky logits make a few keys
dominate each row. Inputs are seeded and synthetic: random Q and K, V = c."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu
import static_triangle_sparse_amd as tsa

pytestmark = pytest.mark.gpu

KW = dict(sink=128, window=2048, last_q=128)
REL_TOL = 1e-4  # relative to max|c|; fp32 accumulation over <= 2^15 terms


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


@pytest.mark.parametrize("peak", [1.0, 6.0])
@pytest.mark.parametrize("mode,split", [("triangle", None), ("triangle", 64), ("causal", None)])
def test_constant_values_come_back(dev, mode, split, peak):
    N, Hq, Hkv, d = 131072, 4, 1, 128
    gu.note(f"constant V N={N} mode={mode} split={split} peak={peak}")
    g = torch.Generator(device="cpu").manual_seed(4242)
    q = (torch.randn(1, Hq, N, d, generator=g) * peak).to(torch.bfloat16).to(dev)
    k = torch.randn(1, Hkv, N, d, generator=g).to(torch.bfloat16).to(dev)
    c = (torch.randn(d, generator=g) * 2.0).to(torch.bfloat16)
    v = c.to(dev).view(1, 1, 1, d).expand(1, Hkv, N, d).contiguous()
    o, lse = tsa.prefill(q, k, v, mode=mode, o_dtype=torch.float32, split=split, **KW)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    cf = c.float().to(dev)
    scale = float(cf.abs().max())
    nq = N // 128
    for t in (0, 1, 40, nq // 2, nq - 2, nq - 1):
        rows = slice(t * 128, (t + 1) * 128)
        err = float((o[:, :, rows] - cf).abs().max()) / scale
        gu.note(f"  tile {t}: max|o - c| / max|c| = {err:.2e}")
        assert err <= REL_TOL, f"tile {t}: output weights do not sum to one ({err:.2e})"
