"""GPU parity of the gfx950 kernel (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TRI = dict(sink=64, window=128, last_q=64)  # the 512-token single-head case


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


# ------------------------------------------------------------ small full cases

@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", ["triangle", "causal"])
def test_single_head_512(dev, mode, o_dtype):
    gu.note(f"single head N=512 d=64 mode={mode} o={o_dtype}")
    bits, (q, k, v) = gu.make_inputs(0, 1, 1, 1, 512, 64, dev)
    o, lse = gu.run(q, k, v, mode, o_dtype=o_dtype, **TRI)
    ro, rl = gu.oracle(bits, mode, **TRI)
    gu.check(o, lse, ro, rl, f"N=512 {mode}")


SWEEP = [(N, d, hq, hkv) for N in (1, 63, 64, 65, 127, 129, 200, 1000) for d in (64, 128)
         for hq, hkv in ((1, 1), (4, 1), (7, 7))]


@pytest.mark.parametrize("N,d,hq,hkv", SWEEP)
def test_tiny_shape_sweep(dev, N, d, hq, hkv):
    gu.note(f"sweep N={N} d={d} hq={hq} hkv={hkv}")
    bits, (q, k, v) = gu.make_inputs(N * 31 + d + hq, 1, hq, hkv, N, d, dev)
    kw = dict(sink=5, window=70, last_q=33)
    for mode in ("triangle", "causal"):
        o, lse = gu.run(q, k, v, mode, **kw)
        ro, rl = gu.oracle(bits, mode, **kw)
        gu.check(o, lse, ro, rl, f"N={N} d={d} {mode}")


def test_batch_two_gqa_seven(dev):
    gu.note("batch 2, 14 q heads / 2 kv heads, N=700, d=128, bf16 out")
    bits, (q, k, v) = gu.make_inputs(7, 2, 14, 2, 700, 128, dev)
    kw = dict(sink=16, window=200, last_q=100)
    for mode in ("triangle", "causal"):
        o, lse = gu.run(q, k, v, mode, o_dtype=torch.bfloat16, **kw)
        ro, rl = gu.oracle(bits, mode, **kw)
        gu.check(o, lse, ro, rl, mode)


@pytest.mark.parametrize("sink,window,last_q", [
    (0, 1, 0),            # each row sees only itself
    (0, 100, 0),          # plain sliding window
    (300, 10, 0),         # sink wider than the window
    (0, 5000, 0),         # window >= N: causal
    (3, 2, 5000),         # last_q >= N: causal
    (1, 1, 1),
    (129, 65, 127),       # nothing tile-aligned
])
def test_edge_parameters(dev, sink, window, last_q):
    gu.note(f"edge sink={sink} window={window} last_q={last_q}")
    N = 1100
    bits, (q, k, v) = gu.make_inputs(sink * 7 + window + last_q, 1, 4, 2, N, 128, dev)
    o, lse = gu.run(q, k, v, "triangle", sink=sink, window=window, last_q=last_q)
    ro, rl = gu.oracle(bits, "triangle", sink, window, last_q)
    gu.check(o, lse, ro, rl, "edge")


def test_strided_token_major_layout(dev):
    gu.note("token-major [B, N, H, d] storage with head stride d")
    N, d = 600, 128
    bits, (q, k, v) = gu.make_inputs(21, 1, 8, 2, N, d, dev)
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)   # strides (.., d, H*d, 1)
    kt = k.transpose(1, 2).contiguous().transpose(1, 2)
    vt = v.transpose(1, 2).contiguous().transpose(1, 2)
    out = torch.empty(1, N, 8, d, dtype=torch.float32, device=dev).transpose(1, 2)
    kw = dict(sink=8, window=128, last_q=64)
    o, lse = tsa.prefill(qt, kt, vt, "triangle", out=out, **kw)
    torch.cuda.synchronize()
    ro, rl = gu.oracle(bits, "triangle", **kw)
    gu.check(o, lse, ro, rl, "strided")


# ------------------------------------------------------- closed forms, invariants

def test_zero_queries_give_log_count(dev):
    gu.note("q = 0 closed form, N=3000")
    N, sink, window, last_q = 3000, 100, 300, 200
    bits, (q, k, v) = gu.make_inputs(3, 1, 2, 1, N, 128, dev)
    q.zero_()
    _, lse = gu.run(q, k, v, "triangle", sink=sink, window=window, last_q=last_q)
    i = np.arange(N)
    count = np.where((i >= N - last_q) | (i < window), i + 1, window + np.minimum(sink, i + 1 - window))
    got = lse[0].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - np.log(count)[None])) < 2e-5


def test_skipped_tiles_are_never_read(dev):
    # NaN in every key tile a query tile does not keep leaves that query
    # tile's rows finite and bit-identical.
    gu.note("NaN poison of skipped tiles, N=8192")
    N = 8192
    kw = dict(sink=128, window=2048, last_q=0)
    bits, (q, k, v) = gu.make_inputs(4, 1, 4, 1, N, 128, dev)
    o_ref, l_ref = gu.run(q, k, v, "triangle", o_dtype=torch.bfloat16, **kw)
    plan = tsa.device_plan(N, "triangle", device=dev, **kw)
    t = 40
    kept = set(plan.k_tile[plan.row_ptr[t]:plan.row_ptr[t + 1]].tolist())
    k2, v2 = k.clone(), v.clone()
    for kt in range(N // 64):
        if kt not in kept:
            k2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
            v2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
    o2, l2 = gu.run(q, k2, v2, "triangle", o_dtype=torch.bfloat16, **kw)
    rows = slice(t * 128, (t + 1) * 128)
    assert torch.isfinite(o2[:, :, rows]).all()
    assert torch.equal(o2[:, :, rows], o_ref[:, :, rows])
    assert torch.equal(l2[:, :, rows], l_ref[:, :, rows])


def test_runs_are_bit_identical(dev):
    gu.note("determinism, N=5000")
    bits, (q, k, v) = gu.make_inputs(5, 1, 8, 2, 5000, 128, dev)
    for mode in ("triangle", "causal"):
        a = gu.run(q, k, v, mode, sink=128, window=1024, last_q=128, o_dtype=torch.bfloat16)
        b = gu.run(q, k, v, mode, sink=128, window=1024, last_q=128, o_dtype=torch.bfloat16)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_triangle_rows_equal_dense_rows(dev):
    # rows inside their first window and the last-Q rows walk the same tiles in
    # both kernels, so they agree bit for bit
    gu.note("cross-kernel row identity, N=6000")
    N, window, last_q = 6000, 1024, 256
    bits, (q, k, v) = gu.make_inputs(6, 1, 4, 1, N, 128, dev)
    ot, lt = gu.run(q, k, v, "triangle", sink=64, window=window, last_q=last_q)
    oc, lc = gu.run(q, k, v, "causal")
    first = (window // 128) * 128           # whole query tiles inside the window
    last = ((N - last_q + 127) // 128) * 128  # whole query tiles of last-Q rows
    for sl in (slice(0, first), slice(last, N)):
        assert torch.equal(ot[:, :, sl], oc[:, :, sl]) and torch.equal(lt[:, :, sl], lc[:, :, sl])


def test_causal_plan_equals_dense_kernel(dev):
    gu.note("planned causal list vs in-kernel causal range, N=3333")
    N = 3333
    bits, (q, k, v) = gu.make_inputs(8, 1, 4, 2, N, 64, dev)
    oc, lc = gu.run(q, k, v, "causal")
    plan = tsa.device_plan(N, "causal", device=dev)
    o = torch.empty_like(oc)
    lse = torch.empty_like(lc)
    t = tsa.make_tensors(q, k, v, o, lse)
    tsa.tri_attn_prefill(t, plan.mp, plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                         plan.d_flags.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)


@pytest.mark.parametrize("qscale", [8.0, 16.0])
def test_peaky_softmax(dev, qscale):
    # large logits and planted spike keys in the sink, window and last-Q
    # regions exercise the running-max rescale
    gu.note(f"peaky softmax qscale={qscale}")
    N, d = 2500, 128
    kw = dict(sink=64, window=512, last_q=128)
    bits, _ = gu.make_inputs(9, 1, 2, 1, N, d, dev)
    qb, kb, vb = bits
    qf = gu.as_f64(qb) * qscale
    kf = gu.as_f64(kb)
    rng = np.random.default_rng(10)
    for j in (3, 40, 700, 1500, 2000, 2450):
        kf[0, 0, j] = 0.5 * qf[0, 0, min(N - 1, j + int(rng.integers(0, 200)))] / qscale * 4
    import synth
    qb2 = synth.f32_to_bf16_bits(qf.astype(np.float32))
    kb2 = synth.f32_to_bf16_bits(kf.astype(np.float32))
    bits2 = (qb2, kb2, vb)
    q, k, v = (gu.bits_to_device(x, dev) for x in bits2)
    for mode in ("triangle", "causal"):
        o, lse = gu.run(q, k, v, mode, **kw)
        ro, rl = gu.oracle(bits2, mode, **kw)
        gu.check(o, lse, ro, rl, f"peaky {mode}")


def test_custom_softmax_scale(dev):
    gu.note("custom scale 0.05")
    bits, (q, k, v) = gu.make_inputs(11, 1, 2, 2, 900, 64, dev)
    kw = dict(sink=32, window=256, last_q=64)
    o, lse = gu.run(q, k, v, "triangle", scale=0.05, **kw)
    ro, rl = gu.oracle(bits, "triangle", scale=0.05, **kw)
    gu.check(o, lse, ro, rl, "scale")
