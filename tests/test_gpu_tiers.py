"""GPU parity of the precision tiers (TriAttention page: tiles scored at two
precisions chosen by per-head diagonal-distance boundaries, combined in one
normalised output; here fp8 e4m3 scores on far tiles): the fp8 copy of K
bit for bit against the oracle's quantization, and the tiered layer against
oracle/tiers.py, which scores far tiles from the same fp8 values."""
import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
import synth
from oracle import tiers as otiers
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


def _codes(values):
    """e4m3 codes of values that are exactly e4m3 (the oracle's outputs).  A
    zero maps to code 0: +0 and -0 (0x80) are the same value, and which of
    the two a rounding to zero yields is not part of what the method fixes."""
    table = otiers.e4m3_values()
    pos = table[:127]                       # codes 0x00..0x7E, increasing
    a = np.abs(values)
    idx = np.searchsorted(pos, a)
    assert np.all(pos[np.minimum(idx, 126)] == a), "not an e4m3 value"
    return np.where((values < 0), idx | 0x80, idx).astype(np.uint8)


def _permute_row(d):
    """channel of byte p of a stored row (the kernel's operand order)"""
    p = np.arange(d)
    s, h, j = p // 64, (p // 32) % 2, p % 32
    return 64 * s + 16 * (j // 8) + 8 * h + j % 8


@pytest.mark.parametrize("N,d,B,Hkv", [(1000, 128, 1, 2), (333, 64, 2, 1)])
def test_fp8_k_matches_the_oracle_quantization(dev, N, d, B, Hkv):
    gu.note(f"fp8 K quantization N={N} d={d} B={B} Hkv={Hkv}")
    bits, (q, k, v) = gu.make_inputs(60 + N, B, Hkv, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k)
    torch.cuda.synchronize()
    kf = gu.as_f64(bits[1])
    nh = -(-N // 64)
    k8 = qk.k8[:B * Hkv * N * d].cpu().numpy().reshape(B, Hkv, N, d)
    sc = qk.scale[:B * Hkv * nh].cpu().numpy().reshape(B, Hkv, nh)
    perm = _permute_row(d)
    for b in range(B):
        for g in range(Hkv):
            for hb in range(nh):
                blk = kf[b, g, hb * 64:min(N, hb * 64 + 64)]
                vals, s = otiers.quantize(blk)
                assert sc[b, g, hb] == s, (b, g, hb)
                want = _codes(vals)[:, perm]
                got = k8[b, g, hb * 64:min(N, hb * 64 + 64)].copy()
                got[got == 0x80] = 0
                assert np.array_equal(got, want), (b, g, hb)


CASES = [  # N, d, Hq, Hkv, sink, window, last_q, low_dist per head
    (1000, 128, 4, 2, 64, 512, 64, [0, 128, 300, 10 ** 6]),
    (700, 64, 2, 1, 32, 300, 0, [-63, 100]),
    (129, 128, 2, 2, 16, 64, 32, [0, 0]),
]


@pytest.mark.parametrize("N,d,Hq,Hkv,sink,window,last_q,dist", CASES)
def test_tiered_layer_matches_the_oracle(dev, N, d, Hq, Hkv, sink, window, last_q, dist):
    gu.note(f"tiered layer N={N} d={d} Hq={Hq} dist={dist}")
    bits, (q, k, v) = gu.make_inputs(70 + N, 1, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k)
    o = torch.full((1, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((1, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="tiered", sink=sink, window=window, last_q=last_q, plan=qk,
                low_dist=dist, o_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    ro, rl = otiers.attention(qf, kf, vf, sink, window, last_q, dist)
    err, rel = gu.check(o, lse, ro, rl, f"tiered N={N}")
    gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")


def test_no_low_tiles_is_bit_identical_to_the_triangle_kernel(dev):
    gu.note("tiered layer with boundaries past N vs tri_attn_prefill, N=1500")
    N = 1500
    _, (q, k, v) = gu.make_inputs(91, 1, 4, 2, N, 128, dev)
    qk = tsa.quantize_k(q, k)
    kw = dict(sink=64, window=256, last_q=64)
    o = torch.empty((1, 4, N, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, 4, N), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="tiered", plan=qk, low_dist=[N + 1] * 4, o_dtype=torch.bfloat16,
                out=o, lse=lse, **kw)
    ot, lt = gu.run(q, k, v, "triangle", o_dtype=torch.bfloat16, **kw)
    assert torch.equal(o, ot) and torch.equal(lse, lt)


def test_llama_128k_tiered_sampled(dev):
    # far tiles (distance >= 1024 keys) in fp8 on the 128K Llama-shaped layer
    N, Hq, Hkv, d = 131072, 32, 8, 128
    kw = dict(sink=128, window=2048, last_q=128)
    gu.note("tiered 128K: inputs, quantize, layer")
    bits, (q, k, v) = gu.make_inputs(0, 1, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k)
    o = torch.empty((1, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="tiered", plan=qk, low_dist=[1024] * Hq, o_dtype=torch.bfloat16,
                out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in (0, 17, 500)] +
                          [np.arange(N - 64, N)])
    for h in (0, 13, 31):
        g = h // 4
        gu.note(f"  head {h}: oracle on {rows.size} rows")
        ro, rl = otiers.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], kw["sink"],
                                  kw["window"], kw["last_q"], [1024], rows=rows)
        idx = torch.from_numpy(rows).to(dev)
        gu.check(o[:, h:h + 1][:, :, idx], lse[:, h:h + 1][:, :, idx], ro, rl, f"128K head {h}")


def test_tiered_skips_tiles_and_is_deterministic(dev):
    # NaN in every key tile query tile 40 does not keep (K and V, so the fp8
    # copy of those key tiles holds NaN scales and codes) leaves that tile's
    # rows bit-identical; two runs agree bit for bit
    gu.note("tiered: NaN poison of skipped tiles and determinism, N=8192")
    N, Hq = 8192, 4
    kw = dict(sink=128, window=2048, last_q=0)
    dist = [0, 512, 1024, 10 ** 6]
    _, (q, k, v) = gu.make_inputs(41, 1, Hq, 1, N, 128, dev)

    def run(k_, v_):
        qk = tsa.quantize_k(q, k_)
        o = torch.empty((1, Hq, N, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
        tsa.prefill(q, k_, v_, mode="tiered", plan=qk, low_dist=dist, o_dtype=torch.bfloat16, out=o,
                    lse=lse, **kw)
        torch.cuda.synchronize()
        return o, lse
    o_ref, l_ref = run(k, v)
    o_b, l_b = run(k, v)
    assert torch.equal(o_ref, o_b) and torch.equal(l_ref, l_b)
    plan = tsa.device_plan(N, "triangle", device=dev, **kw)
    t = 40
    kept = set(plan.k_tile[plan.row_ptr[t]:plan.row_ptr[t + 1]].tolist())
    k2, v2 = k.clone(), v.clone()
    for kt in range(N // 64):
        if kt not in kept:
            k2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
            v2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
    o2, l2 = run(k2, v2)
    rows = slice(t * 128, (t + 1) * 128)
    assert torch.isfinite(o2[:, :, rows]).all()
    assert torch.equal(o2[:, :, rows], o_ref[:, :, rows]) and torch.equal(l2[:, :, rows], l_ref[:, :, rows])


# ----------------------------------------------------------------- fp4 tier

def _codes4(values):
    """e2m1 codes of values that are exactly e2m1 (the oracle's outputs); a
    zero maps to code 0 (+0 and -0 are the same value)."""
    pos = otiers.e2m1_values()[:8]                 # codes 0..7, increasing
    a = np.abs(values)
    idx = np.searchsorted(pos, a)
    assert np.all(pos[np.minimum(idx, 7)] == a), "not an e2m1 value"
    return np.where(values < 0, idx | 8, idx).astype(np.uint8)


@pytest.mark.parametrize("N,d,B,Hkv", [(1000, 128, 1, 2), (333, 64, 2, 1)])
def test_fp4_k_matches_the_oracle_quantization(dev, N, d, B, Hkv):
    gu.note(f"fp4 K quantization N={N} d={d} B={B} Hkv={Hkv}")
    bits, (q, k, v) = gu.make_inputs(80 + N, B, Hkv, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    torch.cuda.synchronize()
    kf = gu.as_f64(bits[1])
    nh = -(-N // 64)
    raw = qk.k4[:B * Hkv * N * d // 2].cpu().numpy().reshape(B, Hkv, N, d // 2)
    nib = np.stack([raw & 0xF, raw >> 4], axis=-1).reshape(B, Hkv, N, d)   # element order of the row
    sc = qk.scale4[:B * Hkv * nh].cpu().numpy().reshape(B, Hkv, nh)
    perm = _permute_row(d)      # element p of a row (32 per lane half) holds the same channel as byte p of fp8
    for b in range(B):
        for g in range(Hkv):
            for hb in range(nh):
                rows = slice(hb * 64, min(N, hb * 64 + 64))
                vals, s = otiers.quantize4(kf[b, g, rows])
                assert sc[b, g, hb] == s, (b, g, hb)
                got = nib[b, g, rows].copy()
                got[got == 8] = 0
                assert np.array_equal(got, _codes4(vals)[:, perm]), (b, g, hb)


CASES4 = [  # N, d, Hq, Hkv, sink, window, last_q, fp8 boundary, fp4 boundary (per head)
    (1000, 128, 4, 2, 64, 512, 64, [0, 0, 128, 10 ** 6], [256, 10 ** 6, 300, 10 ** 6]),
    (700, 64, 2, 1, 32, 300, 0, [-63, 10 ** 6], [100, -63]),
    (129, 128, 2, 2, 16, 64, 32, [0, 0], [0, 64]),
]


@pytest.mark.parametrize("N,d,Hq,Hkv,sink,window,last_q,dist8,dist4", CASES4)
def test_three_tier_layer_matches_the_oracle(dev, N, d, Hq, Hkv, sink, window, last_q, dist8, dist4):
    gu.note(f"three tiers N={N} d={d} Hq={Hq} fp8 {dist8} fp4 {dist4}")
    bits, (q, k, v) = gu.make_inputs(90 + N, 1, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    o = torch.full((1, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((1, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="tiered", sink=sink, window=window, last_q=last_q, plan=qk,
                low_dist=dist8, fp4_dist=dist4, o_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    ro, rl = otiers.attention(qf, kf, vf, sink, window, last_q, dist8, dist4=dist4)
    err, rel = gu.check(o, lse, ro, rl, f"three tiers N={N}")
    gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")


def test_three_tiers_batch_two_and_seven_heads_per_kv_head(dev):
    # batch 2 (the K copies and scales are per (batch, KV head)) and the
    # Qwen2.5-7B grouping of seven query heads per KV head, each head with its
    # own pair of boundaries
    N, d, B, Hq, Hkv = 600, 128, 2, 7, 1
    dist8 = [0, 64, 10 ** 6, -63, 128, 0, 256]
    dist4 = [256, 10 ** 6, 0, 192, 10 ** 6, 64, 320]
    gu.note(f"three tiers N={N} B={B} Hq={Hq} Hkv={Hkv}")
    bits, (q, k, v) = gu.make_inputs(95, B, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    kw = dict(sink=64, window=200, last_q=100)
    tsa.prefill(q, k, v, mode="tiered", plan=qk, low_dist=dist8, fp4_dist=dist4, o_dtype=torch.float32,
                out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    ro, rl = otiers.attention(qf, kf, vf, kw["sink"], kw["window"], kw["last_q"], dist8, dist4=dist4)
    err, rel = gu.check(o, lse, ro, rl, "three tiers B=2 G=7")
    gu.note(f"  max|dO|={err:.2e} max rel dLSE={rel:.2e}")


def test_unreached_fp4_boundary_is_bit_identical_to_two_tiers(dev):
    gu.note("fp4 boundary past N vs the two-tier layer, N=1500")
    N = 1500
    _, (q, k, v) = gu.make_inputs(93, 1, 4, 2, N, 128, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    kw = dict(sink=64, window=512, last_q=64)
    outs = []
    for fp4 in (None, [N + 1] * 4):
        o = torch.empty((1, 4, N, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, 4, N), dtype=torch.float32, device=dev)
        tsa.prefill(q, k, v, mode="tiered", plan=qk, low_dist=[0, 128, 256, 1024], fp4_dist=fp4,
                    o_dtype=torch.bfloat16, out=o, lse=lse, **kw)
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_three_tiers_skip_tiles_and_are_deterministic(dev):
    gu.note("three tiers: NaN poison of skipped tiles and determinism, N=8192")
    N, Hq = 8192, 4
    kw = dict(sink=128, window=2048, last_q=0)

    def run(k_, v_):
        qk = tsa.quantize_k(q, k_, fp4=True)
        o = torch.empty((1, Hq, N, 128), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
        tsa.prefill(q, k_, v_, mode="tiered", plan=qk, low_dist=[0, 256, 512, 10 ** 6],
                    fp4_dist=[1024, 512, 10 ** 6, 0], o_dtype=torch.bfloat16, out=o, lse=lse, **kw)
        torch.cuda.synchronize()
        return o, lse
    _, (q, k, v) = gu.make_inputs(51, 1, Hq, 1, N, 128, dev)
    o_ref, l_ref = run(k, v)
    o_b, l_b = run(k, v)
    assert torch.equal(o_ref, o_b) and torch.equal(l_ref, l_b)
    plan = tsa.device_plan(N, "triangle", device=dev, **kw)
    t = 40
    kept = set(plan.k_tile[plan.row_ptr[t]:plan.row_ptr[t + 1]].tolist())
    k2, v2 = k.clone(), v.clone()
    for kt in range(N // 64):
        if kt not in kept:
            k2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
            v2[:, :, kt * 64:(kt + 1) * 64] = float("nan")
    o2, l2 = run(k2, v2)
    rows = slice(t * 128, (t + 1) * 128)
    assert torch.isfinite(o2[:, :, rows]).all()
    assert torch.equal(o2[:, :, rows], o_ref[:, :, rows]) and torch.equal(l2[:, :, rows], l_ref[:, :, rows])


def test_llama_128k_three_tiers_sampled(dev):
    # fp8 everywhere off the diagonal band, fp4 from 1024 keys away
    N, Hq, Hkv, d = 131072, 32, 8, 128
    kw = dict(sink=128, window=2048, last_q=128)
    gu.note("three tiers 128K: inputs, quantize, layer")
    bits, (q, k, v) = gu.make_inputs(0, 1, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    o = torch.empty((1, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    tsa.prefill(q, k, v, mode="tiered", plan=qk, low_dist=[0] * Hq, fp4_dist=[1024] * Hq,
                o_dtype=torch.bfloat16, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in (0, 17, 500)] + [np.arange(N - 64, N)])
    for h in (0, 13, 31):
        g = h // 4
        gu.note(f"  head {h}: oracle on {rows.size} rows")
        ro, rl = otiers.attention(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], kw["sink"], kw["window"],
                                  kw["last_q"], [0], rows=rows, dist4=[1024])
        idx = torch.from_numpy(rows).to(dev)
        gu.check(o[:, h:h + 1][:, :, idx], lse[:, h:h + 1][:, :, idx], ro, rl, f"128K three tiers head {h}")


def test_three_tiers_batched(dev):
    # batch entries address the fp8 / fp4 copies and scales by (batch, KV head)
    gu.note("three tiers, batch 2, N=600, d=64")
    B, Hq, Hkv, N, d = 2, 4, 2, 600, 64
    bits, (q, k, v) = gu.make_inputs(97, B, Hq, Hkv, N, d, dev)
    qk = tsa.quantize_k(q, k, fp4=True)
    o = torch.full((B, Hq, N, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=dev)
    dist8, dist4 = [0, 64, 128, 10 ** 6], [256, 10 ** 6, 128, 0]
    tsa.prefill(q, k, v, mode="tiered", sink=32, window=256, last_q=64, plan=qk, low_dist=dist8,
                fp4_dist=dist4, o_dtype=torch.float32, out=o, lse=lse)
    torch.cuda.synchronize()
    qf, kf, vf = (gu.as_f64(x) for x in bits)
    ro, rl = otiers.attention(qf, kf, vf, 32, 256, 64, dist8, dist4=dist4)
    gu.check(o, lse, ro, rl, "three tiers batched")
