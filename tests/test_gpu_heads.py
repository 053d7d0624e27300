"""GPU parity of the triangle layer with per-head boundaries (TriAttention
page: each head's region encoded by diagonal-distance boundaries; here each
query head has its own sink and window): every head against the oracle's
triangle attention with that head's (sink, window), and bit-identity with
the single-boundary kernel when all heads share one pair."""
import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


def run_heads(q, k, v, plan, o_dtype=torch.float32):
    B, Hq, N, d = q.shape
    o = torch.full((B, Hq, N, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    tsa.prefill(q, k, v, mode="triangle_heads", plan=plan, o_dtype=o_dtype, out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("N,d,B,Hq,Hkv,last_q", [(1500, 128, 2, 6, 2, 100), (700, 64, 1, 4, 4, 0),
                                                 (129, 128, 1, 3, 1, 64), (1, 64, 1, 2, 1, 0)])
def test_each_head_matches_its_own_triangle(dev, N, d, B, Hq, Hkv, last_q):
    gu.note(f"per-head boundaries N={N} d={d} B={B} Hq={Hq} Hkv={Hkv} last_q={last_q}")
    pairs = [(0, 1), (128, 256), (16, 1000), (N + 3, 5), (3, 70), (64, N + 1)][:Hq]
    sink = [s for s, _ in pairs]
    window = [w for _, w in pairs]
    bits, (q, k, v) = gu.make_inputs(40 + N, B, Hq, Hkv, N, d, dev)
    plan = tsa.head_plan(N, sink, window, last_q, dev)
    o, lse = run_heads(q, k, v, plan)
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    from oracle import attention as oatt
    G = Hq // Hkv
    for h, (s, w) in enumerate(pairs):
        g = h // G
        ro, rl = oatt.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], "triangle", s, w, last_q)
        gu.check(o[:, h:h + 1], lse[:, h:h + 1], ro, rl, f"head {h} sink={s} window={w}")


def test_shared_boundaries_are_bit_identical_to_the_single_plan(dev):
    gu.note("per-head boundaries, all heads equal, vs tri_attn_prefill, N=2000")
    N, Hq = 2000, 8
    _, (q, k, v) = gu.make_inputs(77, 1, Hq, 2, N, 128, dev)
    plan = tsa.head_plan(N, [128] * Hq, [512] * Hq, 128, dev)
    o, lse = run_heads(q, k, v, plan, torch.bfloat16)
    ot, lt = gu.run(q, k, v, "triangle", sink=128, window=512, last_q=128, o_dtype=torch.bfloat16)
    assert torch.equal(o, ot) and torch.equal(lse, lt)


def test_llama_128k_per_head_windows_sampled(dev):
    # 32 heads, windows 512 .. 4096 and sinks 0 / 128 alternating, last-Q 128
    N, Hq, Hkv, d = 131072, 32, 8, 128
    window = [512 << (h % 4) for h in range(Hq)]
    sink = [128 * (h % 2) for h in range(Hq)]
    gu.note("per-head boundaries 128K: inputs and plan")
    bits, (q, k, v) = gu.make_inputs(5, 1, Hq, Hkv, N, d, dev)
    plan = tsa.head_plan(N, sink, window, 128, dev)
    o, lse = run_heads(q, k, v, plan, torch.bfloat16)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    from oracle import attention as oatt
    rows = gu.sample_rows(N, seed=3)
    idx = torch.from_numpy(rows).to(dev)
    for h in (0, 5, 10, 31):
        g = h // 4
        gu.note(f"  head {h}: sink {sink[h]} window {window[h]}, oracle on {rows.size} rows")
        ro, rl = oatt.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], "triangle", sink[h],
                                window[h], 128, rows=rows)
        gu.check(o[:, h:h + 1][:, :, idx], lse[:, h:h + 1][:, :, idx], ro, rl, f"128K head {h}")


def test_per_head_skips_tiles_and_is_deterministic(dev):
    # heads of one KV group with different windows: NaN in every key tile that
    # no head of the group keeps for query tile 40 leaves that tile's rows of
    # every head bit-identical; two runs agree bit for bit
    gu.note("per-head: NaN poison of skipped tiles and determinism, N=8192")
    N, Hq = 8192, 4
    sink, window = [0, 128, 0, 128], [256, 512, 1024, 2048]
    _, (q, k, v) = gu.make_inputs(47, 1, Hq, 1, N, 128, dev)
    plan = tsa.head_plan(N, sink, window, 0, dev)
    o_ref, l_ref = run_heads(q, k, v, plan, torch.bfloat16)
    o_b, l_b = run_heads(q, k, v, plan, torch.bfloat16)
    assert torch.equal(o_ref, o_b) and torch.equal(l_ref, l_b)
    nq = N // 128
    t = 40
    kept = set()
    for h in range(Hq):
        r = h * nq + t
        kept |= set(plan.k_tile[plan.row_ptr[r]:plan.row_ptr[r + 1]].tolist())
    k2, v2 = k.clone(), v.clone()
    for kt in range(N // 64):
        if kt not in kept:
            k2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
            v2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
    o2, l2 = run_heads(q, k2, v2, plan, torch.bfloat16)
    rows = slice(t * 128, (t + 1) * 128)
    assert torch.isfinite(o2[:, :, rows]).all()
    assert torch.equal(o2[:, :, rows], o_ref[:, :, rows]) and torch.equal(l2[:, :, rows], l_ref[:, :, rows])
