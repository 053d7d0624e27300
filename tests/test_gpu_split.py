"""GPU parity of the split launch (tri_attn_prefill_split): the last-Q query
tiles' lists walked in chunks on separate workgroups, partial softmax sums
merged.  The layer is the triangle layer (TriangleMix pages: sink, window and
last-Q regions), so the oracle is oracle/attention.py (per head for per-head
boundaries); rows outside the split tiles run the unsplit code on the same
lists and must equal tri_attn_prefill bit for bit."""
import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
import synth
from oracle import attention as oatt
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


def run_split(q, k, v, chunk, o_dtype, **kw):
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    tsa.prefill(q, k, v, split=chunk, o_dtype=o_dtype, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    return o, lse


def heavy_rows(N, last_q):
    first = (N - min(last_q, N)) // 128 * 128 if last_q > 0 else N
    return np.arange(first, N)


CASES = [  # B, Hq, Hkv, N, d, sink, window, last_q, chunk, qscale
    (1, 4, 2, 1000, 128, 16, 128, 300, 3, 1.0),
    (2, 2, 1, 700, 64, 32, 256, 64, 2, 8.0),
    (1, 2, 2, 1500, 128, 0, 64, 128, 1, 16.0),
    (1, 3, 1, 129, 128, 8, 32, 129, 1, 1.0),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,sink,window,last_q,chunk,qscale", CASES)
def test_split_layer_matches_the_oracle(dev, B, Hq, Hkv, N, d, sink, window, last_q, chunk, qscale):
    gu.note(f"split N={N} d={d} B={B} Hq={Hq} last_q={last_q} chunk={chunk} qscale={qscale}")
    qb, kb, vb = synth.qkv_bf16_bits(200 + N, B, Hq, Hkv, N, d)
    if qscale != 1.0:
        qb = synth.f32_to_bf16_bits((gu.as_f64(qb) * qscale).astype(np.float32))
    bits = (qb, kb, vb)
    q, k, v = (gu.bits_to_device(x, dev) for x in bits)
    kw = dict(mode="triangle", sink=sink, window=window, last_q=last_q)
    o, lse = run_split(q, k, v, chunk, torch.float32, **kw)
    ro, rl = gu.oracle(bits, "triangle", sink, window, last_q)
    err, rel = gu.check(o, lse, ro, rl, f"split N={N}")
    gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")
    # rows outside the split tiles: the unsplit walk, bit for bit
    ou, lu = gu.run(q, k, v, "triangle", o_dtype=torch.float32, sink=sink, window=window, last_q=last_q)
    rest = N - heavy_rows(N, last_q).size
    assert torch.equal(o[:, :, :rest], ou[:, :, :rest]) and torch.equal(lse[:, :, :rest], lu[:, :, :rest])


def test_split_bf16_output_and_no_last_q(dev):
    gu.note("split bf16 O, N=1000; and last_q=0 (nothing to split) bit-identical to the plain launch")
    bits, (q, k, v) = gu.make_inputs(301, 1, 4, 2, 1000, 128, dev)
    kw = dict(mode="triangle", sink=64, window=256, last_q=200)
    o, lse = run_split(q, k, v, 4, torch.bfloat16, **kw)
    ro, rl = gu.oracle(bits, "triangle", 64, 256, 200)
    gu.check(o, lse, ro, rl, "split bf16")
    kw0 = dict(mode="triangle", sink=64, window=256, last_q=0)
    o0, l0 = run_split(q, k, v, 4, torch.bfloat16, **kw0)
    ou, lu = gu.run(q, k, v, "triangle", o_dtype=torch.bfloat16, sink=64, window=256, last_q=0)
    assert torch.equal(o0, ou) and torch.equal(l0, lu)


def test_split_per_head_plan(dev):
    gu.note("split per-head plan, N=1100, chunk 2")
    N, Hq, Hkv, d = 1100, 4, 2, 128
    sink, window, last_q = [0, 64, 16, 128], [64, 128, 512, 2000], 150
    bits, (q, k, v) = gu.make_inputs(307, 1, Hq, Hkv, N, d, dev)
    hp = tsa.head_plan(N, sink, window, last_q, dev)
    o, lse = run_split(q, k, v, 2, torch.float32, mode="triangle_heads", plan=hp)
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        ro, rl = oatt.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], "triangle",
                                sink[h], window[h], last_q)
        gu.check(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"per-head split h={h}")
    ou = torch.empty_like(o)
    lu = torch.empty_like(lse)
    tsa.prefill(q, k, v, mode="triangle_heads", plan=hp, o_dtype=torch.float32, out=ou, lse=lu)
    torch.cuda.synchronize()
    rest = N - heavy_rows(N, last_q).size
    assert torch.equal(o[:, :, :rest], ou[:, :, :rest]) and torch.equal(lse[:, :, :rest], lu[:, :, :rest])


def test_llama_128k_split_sampled(dev):
    # the 128K Llama-shaped layer with the last-Q tile of every head walked in
    # 32 chunks of 64 key tiles (the configuration the benchmark times)
    N, Hq, Hkv, d = 131072, 32, 8, 128
    kw = dict(mode="triangle", sink=128, window=2048, last_q=128)
    gu.note("split 128K: inputs, launch")
    bits, (q, k, v) = gu.make_inputs(0, 1, Hq, Hkv, N, d, dev)
    o, lse = run_split(q, k, v, 64, torch.bfloat16, **kw)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ou, lu = gu.run(q, k, v, "triangle", o_dtype=torch.bfloat16, sink=128, window=2048, last_q=128)
    assert torch.equal(o[:, :, :N - 128], ou[:, :, :N - 128]) and torch.equal(lse[:, :, :N - 128], lu[:, :, :N - 128])
    rows = np.concatenate([np.arange(0, 64), np.arange(N - 128, N)])
    ro, rl = gu.oracle(bits, "triangle", 128, 2048, 128, rows=rows)
    idx = torch.from_numpy(rows).to(dev)
    err, rel = gu.check(o[:, :, idx], lse[:, :, idx], ro, rl, "128K split")
    gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d,last_q,chunk", [(2, 4, 2, 600, 64, 10 ** 6, 2), (3, 2, 1, 257, 128, 200, 1)])
def test_split_batches_per_head_and_whole_rows(dev, B, Hq, Hkv, N, d, last_q, chunk):
    # last_q >= N makes every query tile a last-Q tile (all rows split)
    gu.note(f"split per-head B={B} N={N} d={d} last_q={last_q} chunk={chunk}")
    sink, window = [0, 32, 64, 7][:Hq], [16, 100, 300, 64][:Hq]
    bits, (q, k, v) = gu.make_inputs(311 + N, B, Hq, Hkv, N, d, dev)
    hp = tsa.head_plan(N, sink, window, last_q, dev)
    o, lse = run_split(q, k, v, chunk, torch.bfloat16, mode="triangle_heads", plan=hp)
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        ro, rl = oatt.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], "triangle",
                                sink[h], window[h], last_q)
        gu.check(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"split B={B} h={h}")


def test_split_skips_tiles_and_is_deterministic(dev):
    gu.note("split: NaN poison of skipped tiles and determinism, N=8192")
    N, Hq = 8192, 4
    kw = dict(mode="triangle", sink=128, window=1024, last_q=128)
    _, (q, k, v) = gu.make_inputs(43, 1, Hq, 1, N, 128, dev)
    o_ref, l_ref = run_split(q, k, v, 16, torch.bfloat16, **kw)
    o_b, l_b = run_split(q, k, v, 16, torch.bfloat16, **kw)
    assert torch.equal(o_ref, o_b) and torch.equal(l_ref, l_b)
    plan = tsa.device_plan(N, "triangle", 128, 1024, 128, dev)
    t = 30
    kept = set(plan.k_tile[plan.row_ptr[t]:plan.row_ptr[t + 1]].tolist())
    k2, v2 = k.clone(), v.clone()
    for kt in range(N // 64):
        if kt not in kept:
            k2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
            v2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
    o2, l2 = run_split(q, k2, v2, 16, torch.bfloat16, **kw)
    rows = slice(t * 128, (t + 1) * 128)
    assert torch.isfinite(o2[:, :, rows]).all()
    assert torch.equal(o2[:, :, rows], o_ref[:, :, rows]) and torch.equal(l2[:, :, rows], l_ref[:, :, rows])
