"""Pins of the dynamic tile-selection oracle (oracle/dynamic.py) against
things other than itself: a scalar brute force, special cases that reduce to
the causal plan or to plain causal attention, closed forms on planted inputs,
invariances the definition implies, and an independent bf16 rounding.

FlashPrefill page: section 2.1 (probe queries, pooled keys), 2.2 (keep a
block when its score reaches alpha times the query block's maximum), 2.3
(walk the kept blocks by index).
"""
import math

import numpy as np
import pytest

import synth
from oracle import attention as oatt
from oracle import brute as obrute
from oracle import dynamic as dyn
from oracle import mask as omask


def _inputs(seed, B, Hq, Hkv, N, d):
    qb, kb, vb = synth.qkv_bf16_bits(seed, B, Hq, Hkv, N, d)
    return synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb)


def _brute_select(q, k, alpha, block_q, block_k, n_probe):
    """Scalar brute force of the selection, loop by loop from the readings."""
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    nq = -(-N // block_q)
    nk = -(-N // block_k)
    lists = {}
    for b in range(B):
        for h in range(Hq):
            g = h // G
            pooled = []
            for kt in range(nk):
                keys = range(kt * block_k, min(N, (kt + 1) * block_k))
                pooled.append([dyn._round_bf16(math.fsum(k[b][g][j][c] for j in keys) / len(keys))
                               .item() for c in range(d)])
            for t in range(nq):
                last = min(N, (t + 1) * block_q) - 1
                cands = list(range(last // block_k + 1))
                probes = [t * block_q + p * (block_q // n_probe) for p in range(n_probe)]
                probes = [i for i in probes if i < N]
                score = [0.0] * len(cands)
                for i in probes:
                    seen = [kt for kt in cands if kt * block_k <= i]
                    z = [scale * math.fsum(q[b][h][i][c] * pooled[kt][c] for c in range(d))
                         for kt in seen]
                    m = max(z)
                    w = [math.exp(x - m) for x in z]
                    tot = math.fsum(w)
                    for kt, x in zip(seen, w):
                        score[kt] += x / tot / len(probes)
                top = max(score)
                kept = []
                for kt in cands:
                    diag = kt * block_k + block_k - 1 > t * block_q
                    near = abs(score[kt] - alpha * top) <= 1e-12 * top
                    kept.append((kt, diag or score[kt] >= alpha * top, near and not diag))
                lists[(b, h, t)] = kept
    return lists


@pytest.mark.parametrize("N,alpha", [(1, 0.5), (40, 0.3), (97, 0.6), (160, 0.9), (160, 1.0)])
def test_select_matches_brute_force(N, alpha):
    q, k, _ = _inputs(3 + N, 1, 2, 1, N, 8)
    q = q * 3.0  # sharper softmax: more tiles fall below the threshold
    row_ptr, k_tile, flags = dyn.select_tiles(q, k, alpha, block_q=32, block_k=16, n_probe=4)
    ref = _brute_select(q.tolist(), k.tolist(), alpha, 32, 16, 4)
    nq = -(-N // 32)
    n_checked = 0
    for (b, h, t), kept in ref.items():
        r = (b * 2 + h) * nq + t
        got = set(k_tile[row_ptr[r]:row_ptr[r + 1]].tolist())
        for kt, keep, near in kept:
            if near:
                continue
            assert (kt in got) == keep, (b, h, t, kt)
            n_checked += 1
    assert n_checked > 0


def test_alpha_zero_is_the_causal_plan():
    # every score is >= 0 = alpha * max: all causal tiles kept, flags as the causal plan
    N = 333
    q, k, _ = _inputs(5, 2, 4, 2, N, 16)
    row_ptr, k_tile, flags = dyn.select_tiles(q, k, 0.0, block_q=64, block_k=32, n_probe=8)
    crp, ckt, cfl = omask.brute_tiles(N, 64, 32, "causal")
    nq = crp.size - 1
    for r in range(2 * 4):
        s, e = row_ptr[r * nq], row_ptr[(r + 1) * nq]
        assert np.array_equal(k_tile[s:e], ckt)
        assert np.array_equal(flags[s:e], cfl)
        assert np.array_equal(row_ptr[r * nq:(r + 1) * nq + 1] - s, crp)


def test_planted_sink_block_alone_survives_a_high_threshold():
    # every query points along channel 0 and so does every key of tile 0; the
    # other keys are small noise: tile 0 dominates every probe's softmax, so
    # with alpha = 0.9 the lists are exactly {0} plus the diagonal tiles
    N, d = 512, 16
    rng = np.random.default_rng(7)
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    q += 0.01 * rng.standard_normal(q.shape)
    k = 0.05 * rng.standard_normal((1, 1, N, d))
    k[0, 0, :64, 0] = 20.0
    row_ptr, k_tile, flags = dyn.select_tiles(q, k, 0.9)
    for t in range(N // 128):
        got = k_tile[row_ptr[t]:row_ptr[t + 1]].tolist()
        diag = [kt for kt in range(2 * t, 2 * t + 2)]
        assert got == sorted(set([0] + diag)), (t, got)


def test_scores_are_a_probability_mass_per_query_tile():
    # each probe's softmax sums to one over the tiles it sees, so their mean does too
    q, k, _ = _inputs(11, 1, 2, 1, 700, 32)
    _, _, _, scores = dyn.select_tiles(q, k, 0.5, return_scores=True)
    for s, thr in scores:
        assert math.isclose(s.sum(), 1.0, rel_tol=0, abs_tol=1e-12)
        assert math.isclose(thr, 0.5 * s.max())


def test_probe_rows():
    assert dyn.probe_rows(0, 1000).tolist() == list(range(0, 128, 8))
    assert dyn.probe_rows(2, 300).tolist() == [256 + 8 * p for p in range(6)]
    assert dyn.probe_rows(0, 1).tolist() == [0]


def test_pooled_keys_closed_form_and_partial_tile():
    # constant keys per tile pool to that constant; the last tile averages
    # only the keys < N
    N, d = 150, 4
    k = np.zeros((1, 1, N, d))
    for kt in range(3):
        k[0, 0, kt * 64:(kt + 1) * 64] = kt + 0.5
    k[0, 0, 128:] = np.arange(22)[:, None] / 32.0
    kb = dyn.pooled_keys(k, 64, to_bf16=False)
    assert np.array_equal(kb[0, 0, :2], np.array([[0.5] * d, [1.5] * d]))
    assert np.allclose(kb[0, 0, 2], np.arange(22).mean() / 32.0, rtol=0, atol=1e-15)


def test_bf16_rounding_agrees_with_the_input_generator():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000).astype(np.float32) * np.float32(3)
    ours = dyn._round_bf16(x.astype(np.float64))
    theirs = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(x))
    assert np.array_equal(ours, theirs)


def test_selection_invariances_of_the_exact_scores():
    # permuting the keys inside each tile, or adding one vector to every key,
    # leaves the (unrounded) tile scores unchanged
    N, d = 400, 16
    q, k, _ = _inputs(13, 1, 1, 1, N, d)
    kb = dyn.pooled_keys(k, 64, to_bf16=False)
    perm = k.copy()
    rng = np.random.default_rng(2)
    for kt in range(-(-N // 64)):
        idx = np.arange(kt * 64, min(N, kt * 64 + 64))
        perm[0, 0, idx] = k[0, 0, rng.permutation(idx)]
    assert np.allclose(dyn.pooled_keys(perm, 64, to_bf16=False), kb, rtol=0, atol=1e-14)
    shift = rng.standard_normal(d)
    kb2 = dyn.pooled_keys(k + shift, 64, to_bf16=False)
    for t in range(4):
        rows = dyn.probe_rows(t, N)
        last = min(N, (t + 1) * 128) - 1
        s1 = dyn.tile_scores(q[0, 0, rows], kb[0, 0], rows, last, 0.25)
        s2 = dyn.tile_scores(q[0, 0, rows], kb2[0, 0], rows, last, 0.25)
        assert np.allclose(s1, s2, rtol=1e-10, atol=1e-14)


def test_attention_over_the_causal_lists_is_causal_attention():
    N = 300
    q, k, v = _inputs(17, 1, 4, 2, N, 16)
    crp, ckt, _ = omask.brute_tiles(N, 128, 64, "causal")
    nq = crp.size - 1
    # the same list for every (batch, head) in one CSR
    row_ptr = [0]
    for r in range(4):
        for t in range(nq):
            row_ptr.append(row_ptr[-1] + crp[t + 1] - crp[t])
    k_tile = np.tile(ckt, 4)
    got = dyn.attention_tiles(q, k, v, np.asarray(row_ptr), k_tile)
    ro, rl = oatt.attention(q, k, v, "causal")
    for h in range(4):
        o, lse = got[(0, h)]
        assert np.allclose(o, ro[0, h], rtol=0, atol=1e-12)
        assert np.allclose(lse, rl[0, h], rtol=0, atol=1e-12)


def test_attention_over_diagonal_lists_matches_brute_force():
    # lists holding only the diagonal tiles: a tile-granular local attention;
    # the scalar brute force with the equivalent key sets agrees
    N, d = 70, 4
    q, k, v = _inputs(19, 1, 1, 1, N, d)
    row_ptr, k_tile, _ = dyn.select_tiles(q * 50, k * 50, 1.0, block_q=32, block_k=16, n_probe=4)
    got = dyn.attention_tiles(q, k, v, row_ptr, k_tile, block_q=32, block_k=16)[(0, 0)]
    nq = -(-N // 32)
    scale = 1.0 / math.sqrt(d)
    for i in range(N):
        t = i // 32
        kts = k_tile[row_ptr[t]:row_ptr[t + 1]]
        js = [j for kt in kts for j in range(kt * 16, kt * 16 + 16) if j <= i and j < N]
        z = [scale * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) for j in js]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        tot = math.fsum(w)
        o = [math.fsum(w[n] * v[0, 0, js[n], c] for n in range(len(js))) / tot for c in range(d)]
        assert np.allclose(got[0][i], o, rtol=0, atol=1e-12)
        assert math.isclose(got[1][i], m + math.log(tot), abs_tol=1e-12)
    assert nq == 3


def test_brute_attention_agrees_on_causal_lists():
    # the list walker and the brute-force attention of the static oracle agree
    N, d = 48, 4
    q, k, v = _inputs(23, 1, 2, 1, N, d)
    crp, ckt, _ = omask.brute_tiles(N, 128, 64, "causal")
    row_ptr = np.array([0, ckt.size, 2 * ckt.size])
    got = dyn.attention_tiles(q, k, v, row_ptr, np.tile(ckt, 2))
    bo, bl = obrute.attention(q.tolist(), k.tolist(), v.tolist(), "causal")
    for h in range(2):
        assert np.allclose(got[(0, h)][0], np.asarray(bo[0][h]), rtol=0, atol=1e-12)
        assert np.allclose(got[(0, h)][1], np.asarray(bl[0][h]), rtol=0, atol=1e-12)


def test_bf16_pooled_keys_move_only_near_threshold_decisions():
    # The pooled keys are rounded to bf16 (the precision the selection's
    # products take them in): a reading of where the decision is taken, not
    # of what is selected.  Against fp64 pooled keys, every tile decided
    # differently must lie within 2% of its threshold, and almost all lists
    # are unchanged.
    q, k, _ = _inputs(77, 1, 4, 2, 3000, 64)
    q = q * 4.0
    rp_b, kt_b, _, sc_b = dyn.select_tiles(q, k, 0.5, return_scores=True)
    rp_f, kt_f, _, sc_f = dyn.select_tiles(q, k, 0.5, return_scores=True, pooled_bf16=False)
    same = 0
    for r in range(rp_b.size - 1):
        a = set(kt_b[rp_b[r]:rp_b[r + 1]].tolist())
        b = set(kt_f[rp_f[r]:rp_f[r + 1]].tolist())
        s, thr = sc_f[r]
        for t in a ^ b:
            assert abs(s[t] - thr) <= 0.02 * thr, (r, t, s[t], thr)
        same += a == b
    assert same >= 0.9 * (rp_b.size - 1)
