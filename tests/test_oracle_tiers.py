"""Pins of the precision-tier oracle (oracle/tiers.py; TriAttention page:
tiles split by per-head diagonal-distance boundaries into precision groups
combined in one softmax): e4m3 rounding against an exhaustive search of the
code table, scale edge cases, the two special cases that reduce to exact
triangle attention, the tile boundary rule, and a scalar brute force."""
import math

import numpy as np
import pytest

import synth
from oracle import attention as oatt
from oracle import tiers


def _nearest_code_value(x, table):
    """Exhaustive: the finite e4m3 value nearest to x, ties to the even code
    (mantissa LSB 0); saturate at +-448."""
    fin = [(c, vv) for c, vv in enumerate(table) if not math.isnan(vv)]
    x = max(-448.0, min(448.0, x))
    best = min(abs(vv - x) for _, vv in fin)
    cands = [(c, vv) for c, vv in fin if abs(vv - x) == best]
    if len(cands) > 1:
        cands = [(c, vv) for c, vv in cands if c % 2 == 0] or cands
    # +0 and -0 tie at zero: either is zero
    return cands[0][1]


def test_round_e4m3_matches_exhaustive_search():
    table = tiers.e4m3_values()
    fin = table[~np.isnan(table)]
    assert np.nanmax(table) == 448.0 and np.min(fin[fin > 0]) == 2.0 ** -9
    rng = np.random.default_rng(4)
    xs = list(rng.standard_normal(3000) * 40) + list(rng.standard_normal(500) * 0.01)
    pos = np.unique(fin[fin >= 0])
    xs += list((pos[1:] + pos[:-1]) / 2)                 # every exact midpoint
    xs += list(-(pos[1:] + pos[:-1]) / 2)
    xs += [0.0, 447.0, 448.0, 449.0, 460.0, 470.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]
    xs = np.asarray(xs, dtype=np.float32).astype(np.float64)
    got = tiers.round_e4m3(xs)
    for x, g in zip(xs, got):
        assert g == _nearest_code_value(float(x), table), x


def test_quantize_scales():
    codes, s = tiers.quantize(np.zeros(16, np.float32))
    assert s == 0 and np.all(codes == 0)
    x = np.array([0.5, -2.0, 1.0, 0.25], np.float32)
    codes, s = tiers.quantize(x)
    assert s == np.float32(2.0) / np.float32(448.0)
    assert codes[1] == -448.0                       # the amax maps to the top code
    assert np.allclose(codes * s, x, rtol=2 ** -3, atol=0)


def test_low_tile_rule():
    # query tile 4 (rows 512..639); key tile 5 ends at key 383: distance 129
    assert tiers.low_tile(4, 5, 129) and not tiers.low_tile(4, 5, 130)
    # key tile 8 (keys 512..575) crosses the diagonal: smallest distance -63
    assert tiers.low_tile(4, 8, -63) and not tiers.low_tile(4, 8, -62)


def _inputs(seed, B, Hq, Hkv, N, d):
    qb, kb, vb = synth.qkv_bf16_bits(seed, B, Hq, Hkv, N, d)
    return synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb)


def test_no_low_tiles_is_the_triangle_attention():
    N = 600
    q, k, v = _inputs(8, 1, 2, 1, N, 16)
    o, l = tiers.attention(q, k, v, 32, 200, 50, [10 ** 9, 10 ** 9])
    ro, rl = oatt.attention(q, k, v, "triangle", 32, 200, 50)
    assert np.allclose(o, ro, rtol=0, atol=1e-12) and np.allclose(l, rl, rtol=0, atol=1e-12)


def test_exactly_representable_inputs_make_fp8_tiles_exact():
    # entries in {-1.75, 0, 1.75} with every row and key tile reaching 1.75:
    # 448 / 1.75 = 256 and 1.75 / 448 = 2^-8 are exact in float32, and every
    # scaled value is +-448 or 0 (exact codes), so the fp8 scores are exact
    N, d = 400, 8
    rng = np.random.default_rng(9)
    q = 1.75 * rng.integers(-1, 2, size=(1, 2, N, d)).astype(np.float64)
    k = 1.75 * rng.integers(-1, 2, size=(1, 1, N, d)).astype(np.float64)
    q[..., 0] = 1.75
    k[..., 0] = -1.75
    v = rng.standard_normal((1, 1, N, d))
    o, l = tiers.attention(q, k, v, 16, 100, 0, [-10 ** 9, -10 ** 9])   # every tile fp8
    ro, rl = oatt.attention(q, k, v, "triangle", 16, 100, 0)
    assert np.allclose(o, ro, rtol=0, atol=1e-12) and np.allclose(l, rl, rtol=0, atol=1e-12)


def test_mixed_tiers_against_a_scalar_brute_force():
    N, d = 300, 8
    q, k, v = _inputs(12, 1, 2, 1, N, d)
    dist = [64, 200]
    o, l = tiers.attention(q, k, v, 8, 150, 20, dist, block_q=32, block_k=16)
    scale = 1.0 / math.sqrt(d)
    for h in range(2):
        for i in (0, 31, 100, 161, 250, 299):
            # keys of the row, straight from the mask definition
            js = [j for j in range(i + 1) if j < 8 or i - j < 150 or i >= N - 20]
            row = np.asarray(q[0, h, i], np.float32)
            amax = np.float32(np.max(np.abs(row)))
            q8 = tiers.round_e4m3((row * (np.float32(448) / amax)).astype(np.float32))
            s_q = float(amax / np.float32(448))
            z = []
            for j in js:
                c0 = (j // 16) * 16                      # its 16-key tile
                blk = np.asarray(k[0, 0, c0:c0 + 16], np.float32)
                bmax = np.float32(np.max(np.abs(blk)))
                k8 = tiers.round_e4m3((np.asarray(k[0, 0, j], np.float32) *
                                       (np.float32(448) / bmax)).astype(np.float32))
                s_k = float(bmax / np.float32(448))
                t, kt = i // 32, j // 16
                if t * 32 - (kt * 16 + 15) >= dist[h]:
                    z.append(scale * s_q * s_k * math.fsum(q8[c] * k8[c] for c in range(d)))
                else:
                    z.append(scale * math.fsum(q[0, h, i, c] * k[0, 0, j, c] for c in range(d)))
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = math.fsum(w)
            ref = [math.fsum(w[n] * v[0, 0, js[n], c] for n in range(len(js))) / tot for c in range(d)]
            assert np.allclose(o[0, h, i], ref, rtol=0, atol=1e-12), (h, i)
            assert math.isclose(l[0, h, i], m + math.log(tot), abs_tol=1e-12)


# ----------------------------------------------------------------- fp4 tier

def _nearest_e2m1(x, table):
    """Exhaustive: the e2m1 value nearest to x, ties to the even code
    (mantissa bit 0); saturate at +-6."""
    x = max(-6.0, min(6.0, x))
    best = min(abs(vv - x) for vv in table)
    cands = [(c, vv) for c, vv in enumerate(table) if abs(vv - x) == best]
    if len(cands) > 1:
        cands = [(c, vv) for c, vv in cands if c % 2 == 0] or cands
    return cands[0][1]


def test_round_e2m1_matches_exhaustive_search():
    table = tiers.e2m1_values()
    assert sorted(set(np.abs(table))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rng = np.random.default_rng(14)
    xs = list(rng.standard_normal(2000) * 3) + list(rng.uniform(-7, 7, 1000))
    pos = np.unique(table[table >= 0])
    xs += list((pos[1:] + pos[:-1]) / 2) + list(-(pos[1:] + pos[:-1]) / 2)   # every midpoint
    xs += [0.0, 5.9, 6.0, 6.1, 7.0, 1e6, -1e6, 1e-8]
    xs = np.asarray(xs, dtype=np.float32).astype(np.float64)
    got = tiers.round_e2m1(xs)
    for x, g in zip(xs, got):
        assert g == _nearest_e2m1(float(x), table), x


def test_quantize4_scales():
    codes, s = tiers.quantize4(np.zeros(8, np.float32))
    assert s == 0 and np.all(codes == 0)
    x = np.array([3.0, -12.0, 6.0, 1.5], np.float32)
    codes, s = tiers.quantize4(x)
    assert s == np.float32(2.0)                      # 12 / 6
    assert list(codes) == [1.5, -6.0, 3.0, 1.0]      # 0.75 is a tie: to the even code, 1.0


def test_fp4_tier_absent_or_unreached_is_the_two_tier_layer():
    N = 500
    q, k, v = _inputs(21, 1, 2, 1, N, 16)
    o2, l2 = tiers.attention(q, k, v, 16, 200, 30, [0, 128])
    o3, l3 = tiers.attention(q, k, v, 16, 200, 30, [0, 128], dist4=[10 ** 9, 10 ** 9])
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_exactly_representable_inputs_make_fp4_tiles_exact():
    # entries in {-a, 0, a} with every row and key tile reaching a: every
    # scaled value is +-6 or 0 (exact codes) and 6 / a, a / 6 are exact for
    # a = 1.5 (4 and 0.25), so the fp4 scores are exact
    N, d = 400, 8
    rng = np.random.default_rng(19)
    a = 1.5
    q = a * rng.integers(-1, 2, size=(1, 2, N, d)).astype(np.float64)
    k = a * rng.integers(-1, 2, size=(1, 1, N, d)).astype(np.float64)
    q[..., 0] = a
    k[..., 0] = -a
    v = rng.standard_normal((1, 1, N, d))
    o, l = tiers.attention(q, k, v, 16, 100, 0, [10 ** 9] * 2, dist4=[-10 ** 9] * 2)   # every tile fp4
    ro, rl = oatt.attention(q, k, v, "triangle", 16, 100, 0)
    assert np.allclose(o, ro, rtol=0, atol=1e-12) and np.allclose(l, rl, rtol=0, atol=1e-12)


def test_three_tiers_against_a_scalar_brute_force():
    N, d = 300, 8
    q, k, v = _inputs(23, 1, 2, 1, N, d)
    dist8, dist4 = [0, 40], [64, 100]
    o, l = tiers.attention(q, k, v, 8, 150, 20, dist8, block_q=32, block_k=16, dist4=dist4)
    scale = 1.0 / math.sqrt(d)

    def q_code(row, top, rnd):
        amax = np.float32(np.max(np.abs(row)))
        return rnd((row * (np.float32(top) / amax)).astype(np.float32)), float(amax / np.float32(top))

    for h in range(2):
        for i in (0, 33, 100, 161, 250, 299):
            js = [j for j in range(i + 1) if j < 8 or i - j < 150 or i >= N - 20]
            row = np.asarray(q[0, h, i], np.float32)
            z = []
            for j in js:
                t, kt = i // 32, j // 16
                dist = t * 32 - (kt * 16 + 15)
                if dist >= dist4[h]:
                    top, rnd = 6.0, tiers.round_e2m1
                elif dist >= dist8[h]:
                    top, rnd = 448.0, tiers.round_e4m3
                else:
                    z.append(scale * math.fsum(q[0, h, i, c] * k[0, 0, j, c] for c in range(d)))
                    continue
                qc, s_q = q_code(row, top, rnd)
                c0 = (j // 16) * 16
                blk = np.asarray(k[0, 0, c0:c0 + 16], np.float32)
                bmax = np.float32(np.max(np.abs(blk)))
                kc = rnd((np.asarray(k[0, 0, j], np.float32) * (np.float32(top) / bmax)).astype(np.float32))
                s_k = float(bmax / np.float32(top))
                z.append(scale * s_q * s_k * math.fsum(qc[c] * kc[c] for c in range(d)))
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = math.fsum(w)
            ref = [math.fsum(w[n] * v[0, 0, js[n], c] for n in range(len(js))) / tot for c in range(d)]
            assert np.allclose(o[0, h, i], ref, rtol=0, atol=1e-12), (h, i)
            assert math.isclose(l[0, h, i], m + math.log(tot), abs_tol=1e-12)
