"""Parity at the full benchmark sizes (Llama-3-8B-shaped layer: 32 query heads,
8 KV heads, head_dim 128; sink 128, window 2048, last-Q 128) in the launch
configuration the benchmark times (bf16 O plus f32 LSE on the current
stream): every row of the 32K and 128K triangle layers against the oracle,
and sampled query tiles of the dense layers (whose rows cost O(N) keys
each) and of the stack layer shapes."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KW = dict(sink=128, window=2048, last_q=128)


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N", [32768, 131072])
def test_llama_triangle_layer_every_row(dev, N):
    gu.note(f"llama triangle layer N={N}, every row: inputs and kernel")
    bits, (q, k, v) = gu.make_inputs(0, 1, 32, 8, N, 128, dev)
    o, lse = gu.run(q, k, v, "triangle", o_dtype=torch.bfloat16, **KW)
    o_h, l_h = o.cpu(), lse.cpu()
    del o, lse, q, k, v
    torch.cuda.empty_cache()
    err, rel = gu.oracle_every_row(bits, "triangle", KW, o_h, l_h, what=f"N={N} triangle")
    gu.note(f"  every row of N={N}: max|dO|={err:.2e} max rel dLSE={rel:.2e}")


@pytest.mark.parametrize("N", [32768, 131072])
def test_llama_layer_sampled_rows(dev, N):
    gu.note(f"llama layer N={N}: generating inputs")
    bits, (q, k, v) = gu.make_inputs(0, 1, 32, 8, N, 128, dev)
    modes = ["triangle", "causal"]
    for mode in modes:
        gu.note(f"llama layer N={N} mode={mode}: kernel")
        o, lse = gu.run(q, k, v, mode, o_dtype=torch.bfloat16, **KW)
        if mode == "triangle":
            rows = gu.sample_rows(N, seed=N)
        else:  # dense rows cost O(N) keys each: a few tiles suffice
            nq = N // 128
            rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in (0, 17, nq // 2, nq - 1)])
        gu.note(f"llama layer N={N} mode={mode}: oracle on {rows.size} rows")
        ro, rl = gu.oracle(bits, mode, rows=rows, **KW)
        idx = torch.from_numpy(rows).to(dev)
        err, rel = gu.check(o[:, :, idx], lse[:, :, idx], ro, rl, f"N={N} {mode}")
        gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")
        # every row written (no NaN left by an unwritten row)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        del o, lse


@pytest.mark.parametrize("N,Hq,Hkv,seed", [(65536, 32, 8, 1012), (131072, 28, 4, 1020)])
def test_stack_layer_shapes_sampled_rows(dev, N, Hq, Hkv, seed):
    # the layer shapes the stack benchmarks run: the Llama-shaped layer at 64K
    # and the Qwen2.5-7B-shaped layer (28 query heads, 4 KV heads: 7 per
    # group) at 128K, triangle and dense, bf16 O as timed
    gu.note(f"stack layer N={N} Hq={Hq} Hkv={Hkv}: generating inputs")
    bits, (q, k, v) = gu.make_inputs(seed, 1, Hq, Hkv, N, 128, dev)
    nq = N // 128
    for mode in ("triangle", "causal"):
        gu.note(f"stack layer N={N} Hq={Hq} mode={mode}: kernel")
        o, lse = gu.run(q, k, v, mode, o_dtype=torch.bfloat16, **KW)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        tiles = (0, 16, nq // 3, nq - 1) if mode == "triangle" else (0, 17, nq - 1)
        rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
        gu.note(f"stack layer N={N} mode={mode}: oracle on {rows.size} rows")
        ro, rl = gu.oracle(bits, mode, rows=rows, **KW)
        idx = torch.from_numpy(rows).to(dev)
        err, rel = gu.check(o[:, :, idx], lse[:, :, idx], ro, rl, f"N={N} Hq={Hq} {mode}")
        gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")
        del o, lse
