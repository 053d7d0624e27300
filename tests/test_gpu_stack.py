"""A short TriangleMix layer stack on the GPU: every layer runs in the mode the
layer policy picks (TriangleMix blog "性能": the first layers dense causal, the
rest triangle; 36kr interview: L_tri_start), through ``stack_prefill`` -- the
runner the stack benchmarks time -- and every row of every layer matches the
oracle in that mode.  Llama-3-8B (32 query / 8 KV heads) and Qwen2.5-7B (28 /
4) head shapes, 4 layers at N = 4096 with the triangle from layer 2 on; the
window (2048) is shorter than N, so a layer run in the wrong mode fails."""
import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KW = dict(sink=128, window=2048, last_q=128)


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (28, 4)])
def test_short_stack_every_layer_in_its_mode(dev, Hq, Hkv):
    N, L, tri_start, d = 4096, 4, 2, 128
    gu.note(f"stack Hq={Hq} Hkv={Hkv}: {L} layers at N={N}, triangle from layer {tri_start}")
    inputs = [gu.make_inputs(3000 + 10 * Hq + l, 1, Hq, Hkv, N, d, dev) for l in range(L)]
    outs = [(torch.full((1, Hq, N, d), float("nan"), dtype=torch.bfloat16, device=dev),
             torch.full((1, Hq, N), float("nan"), dtype=torch.float32, device=dev)) for _ in range(L)]
    descs = [tsa.make_tensors(q, k, v, o, lse) for (_, (q, k, v)), (o, lse) in zip(inputs, outs)]
    modes = tsa.stack_prefill(descs, tri_start, **KW)
    torch.cuda.synchronize()
    assert modes == [tsa.layer_mode(l, tri_start) for l in range(L)] == \
        ["causal", "causal", "triangle", "triangle"]
    rows_differ = None
    for l, ((bits, _), (o, lse)) in enumerate(zip(inputs, outs)):
        ro, rl = gu.oracle(bits, modes[l], **KW)
        err, rel = gu.check(o, lse, ro, rl, f"layer {l} ({modes[l]})")
        gu.note(f"  layer {l} {modes[l]}: max|dO|={err:.2e} max rel dLSE={rel:.2e}")
        if modes[l] == "triangle" and rows_differ is None:
            # the two modes really differ on this input (beyond the bound)
            co, _ = gu.oracle(bits, "causal", **KW)
            rows_differ = int(np.sum(np.max(np.abs(co - ro), axis=-1) > 5e-2))
    assert rows_differ > 1000, rows_differ
