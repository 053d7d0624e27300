"""The TriangleMix layer policy: shallow layers keep dense causal attention,
the rest use the triangle pattern.  The TriangleMix blog ("性能") finds 12
dense layers enough for the Llama-3 models and 20 for Qwen2.5; the 36kr
interview gives the same split for Llama as L_tri_start = 12 (triangle on the
deeper 62.5% of 32 layers).  Checked here: ``layer_mode`` draws exactly that
boundary, and the stack workloads of the benchmark (a 32-layer Llama-3-8B
shape, a 28-layer Qwen2.5-7B shape) use it."""
import pytest

import bench
import static_triangle_sparse_amd as tsa


@pytest.mark.parametrize("layers,tri_start,dense", [(32, 12, 12), (28, 20, 20)])
def test_layer_mode_boundary(layers, tri_start, dense):
    modes = [tsa.layer_mode(l, tri_start) for l in range(layers)]
    assert modes[:dense] == ["causal"] * dense
    assert modes[dense:] == ["triangle"] * (layers - dense)


def test_llama_split_is_the_interview_fraction():
    # triangle attention on 62.5% of the 32 layers (L_tri_start = 12)
    modes = [tsa.layer_mode(l, 12) for l in range(32)]
    assert modes.count("triangle") / 32 == 0.625


@pytest.mark.parametrize("cfg,layers,tri_start,heads", [(4, 32, 12, (32, 8)), (5, 28, 20, (28, 4))])
def test_stack_workloads_use_the_policy(cfg, layers, tri_start, heads):
    c = bench.CONFIGS[cfg]
    assert (c["layers"], c["tri_start"], (c["Hq"], c["Hkv"])) == (layers, tri_start, heads)
    assert (c["sink"], c["window"], c["last_q"], c["d"]) == (128, 2048, 128, 128)


def test_edges():
    assert tsa.layer_mode(0, 0) == "triangle"          # no dense layer
    assert tsa.layer_mode(31, 32) == "causal"          # every layer dense
