"""Pins of the CPU oracle against things other than itself.

Each test ties the oracle to a fact fixed by the pages or by mathematics:
a hand-derived tile grid (tests/golden), a pure-Python brute force, closed
forms (all-zero queries give uniform weights, so lse = ln|K_i|), library
attention (torch's scaled_dot_product_attention / logsumexp in float64) on the
special cases that reduce to textbook causal, sliding-window or sink
attention, and invariants (convex combination, masked-key invariance).  The
mutation tests at the end plant plausible mistakes in the oracle and check
that some pin fails.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import brute as obrute
from oracle import mask as omask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "config1_tiles.txt")


def _rand_qkv(seed, B, Hq, Hkv, N, d, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d)) * scale_q
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    return q, k, v


def _count_closed_form(i, N, sink, window, last_q):
    """|K_i| for the triangle mask, derived by hand: a last-Q row or a row
    still inside its first window keeps all i+1 earlier keys; any other row
    keeps its window plus the sink keys that lie left of the window."""
    if i >= N - last_q or i < window:
        return i + 1
    return window + min(sink, i + 1 - window)


# ---------------------------------------------------------------- tile grids

def _read_golden():
    out = {"triangle": {}, "causal": {}}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, t, *tiles = line.split()
            out[kind][int(t)] = [(int(x[:-1]), omask.FULL if x[-1] == "F" else omask.PARTIAL)
                                 for x in tiles]
    return out


def _as_rows(plan):
    row_ptr, k_tile, flags = plan
    return {t: [(int(k_tile[e]), int(flags[e])) for e in range(row_ptr[t], row_ptr[t + 1])]
            for t in range(len(row_ptr) - 1)}


@pytest.mark.parametrize("enumerator", [omask.brute_tiles, omask.interval_tiles])
def test_golden_config1_tile_grid(enumerator):
    gold = _read_golden()
    for kind in ("triangle", "causal"):
        got = _as_rows(enumerator(512, 128, 64, kind, sink=64, window=128, last_q=64))
        assert got == gold[kind], kind


def test_kept_keys_equals_predicate():
    for N in (1, 2, 7, 33, 64, 100):
        for kind, sink, window, last_q in [("causal", 0, 1, 0), ("triangle", 0, 1, 0),
                                           ("triangle", 3, 5, 2), ("triangle", 10, 4, 0),
                                           ("triangle", 0, 7, 9), ("triangle", 200, 1, 0),
                                           ("triangle", 2, 200, 0), ("triangle", 1, 1, 200)]:
            for i in range(N):
                ref = np.nonzero(omask.allowed(i, np.arange(N), N, kind, sink, window, last_q))[0]
                got = omask.kept_keys(i, N, kind, sink, window, last_q)
                assert np.array_equal(ref, got), (N, kind, sink, window, last_q, i)
                if kind == "triangle":
                    assert got.size == _count_closed_form(i, N, sink, window, last_q)


def test_interval_tiles_equal_brute_tiles():
    rng = np.random.default_rng(1)
    for _ in range(300):
        N = int(rng.integers(1, 200))
        bq = int(rng.choice([1, 3, 16, 32, 64]))
        bk = int(rng.choice([1, 5, 16, 32, 64]))
        kind = "causal" if rng.random() < 0.2 else "triangle"
        sink = int(rng.choice([0, 1, rng.integers(0, 2 * N + 1)]))
        window = int(rng.choice([1, rng.integers(1, 2 * N + 2)]))
        last_q = int(rng.choice([0, 1, rng.integers(0, 2 * N + 1)]))
        a = omask.brute_tiles(N, bq, bk, kind, sink, window, last_q)
        b = omask.interval_tiles(N, bq, bk, kind, sink, window, last_q)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), (N, bq, bk, kind, sink, window, last_q)


def test_tile_count_grows_linearly_in_n():
    # O(N) kept work for the triangle pattern at fixed (sink, window, last_q)
    counts = [omask.interval_tiles(n, 128, 64, "triangle", 128, 2048, 128)[0][-1]
              for n in (16384, 32768, 65536)]
    d1 = counts[1] - counts[0]
    d2 = counts[2] - counts[1]
    assert d2 == 2 * d1           # exact: the per-tile count is constant past the window


# ------------------------------------------------------- oracle vs brute force

@pytest.mark.parametrize("case", [
    ("causal", 0, 1, 0), ("triangle", 2, 3, 2), ("triangle", 0, 1, 0), ("triangle", 5, 2, 0),
    ("triangle", 0, 4, 6), ("triangle", 1, 1, 1), ("triangle", 40, 6, 3), ("triangle", 3, 50, 0),
])
@pytest.mark.parametrize("N,d,Hq,Hkv", [(1, 4, 1, 1), (9, 3, 2, 1), (23, 8, 3, 3), (40, 5, 4, 2)])
def test_numpy_oracle_matches_pure_python(case, N, d, Hq, Hkv):
    kind, sink, window, last_q = case
    q, k, v = _rand_qkv(N * 7 + d, 1, Hq, Hkv, N, d, scale_q=2.0)
    o, lse = oatt.attention(q, k, v, kind, sink, window, last_q, row_block=5)
    ob, lb = obrute.attention(q.tolist(), k.tolist(), v.tolist(), kind, sink, window, last_q)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lb))) < 1e-12


def test_numpy_oracle_batch_and_row_subset():
    q, k, v = _rand_qkv(5, 2, 4, 2, 50, 6)
    o, lse = oatt.attention(q, k, v, "triangle", 3, 7, 5)
    rows = np.array([0, 3, 17, 44, 49])
    o2, l2 = oatt.attention(q, k, v, "triangle", 3, 7, 5, rows=rows)
    assert np.allclose(o[:, :, rows], o2, atol=1e-13, rtol=0)
    assert np.allclose(lse[:, :, rows], l2, atol=1e-13, rtol=0)
    ob, lb = obrute.attention(q[1:].tolist(), k[1:].tolist(), v[1:].tolist(), "triangle", 3, 7, 5)
    assert np.max(np.abs(o[1] - np.array(ob)[0])) < 1e-12
    assert np.max(np.abs(lse[1] - np.array(lb)[0])) < 1e-12


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("N,sink,window,last_q", [(64, 4, 8, 8), (200, 16, 32, 0), (200, 0, 5, 50),
                                                  (130, 40, 10, 3), (30, 0, 100, 0)])
def test_zero_queries_give_uniform_weights(N, sink, window, last_q):
    # q = 0 => every kept score is 0 => weights 1/|K_i|, lse = ln|K_i| and,
    # with V = identity columns, o[i, j] = 1/|K_i| exactly on the kept keys.
    d = N
    q = np.zeros((1, 1, N, d))
    k = np.random.default_rng(0).standard_normal((1, 1, N, d))
    v = np.eye(N)[None, None]
    o, lse = oatt.attention(q, k, v, "triangle", sink, window, last_q)
    for i in range(N):
        c = _count_closed_form(i, N, sink, window, last_q)
        assert abs(lse[0, 0, i] - math.log(c)) < 1e-12
        nz = np.count_nonzero(o[0, 0, i] > 0)
        assert nz == c
        assert np.allclose(o[0, 0, i][o[0, 0, i] > 0], 1.0 / c, atol=1e-15, rtol=0)
        assert not np.any(o[0, 0, i, i + 1:])       # never a future key


def test_single_token_and_first_row():
    q, k, v = _rand_qkv(3, 1, 2, 1, 1, 16)
    for kind in ("causal", "triangle"):
        o, lse = oatt.attention(q, k, v, kind, 0, 1, 0)
        for h in range(2):
            assert np.array_equal(o[0, h, 0], v[0, 0, 0])
            z = float(np.dot(q[0, h, 0], k[0, 0, 0])) / 4.0
            assert abs(lse[0, h, 0] - z) < 1e-12


def test_constant_values_give_constant_output():
    q, k, _ = _rand_qkv(4, 1, 2, 2, 90, 8, scale_q=5.0)
    v = np.full((1, 2, 90, 8), -1.75)
    o, _ = oatt.attention(q, k, v, "triangle", 4, 9, 7)
    assert np.allclose(o, -1.75, atol=1e-13, rtol=0)


# -------------------------------------------- library attention special cases

def _sdpa(q, k, v, mask_bool):
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    qt = torch.from_numpy(q)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask_bool))
    s = (qt @ kt.transpose(-1, -2)) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~torch.from_numpy(mask_bool), float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def _check_sdpa(q, k, v, kind, sink, window, last_q, mask_bool):
    o, lse = oatt.attention(q, k, v, kind, sink, window, last_q)
    ro, rl = _sdpa(q, k, v, mask_bool)
    assert np.max(np.abs(o - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_causal_matches_library_attention():
    N = 150
    q, k, v = _rand_qkv(11, 2, 6, 2, N, 16, scale_q=3.0)
    causal = torch.ones(N, N, dtype=torch.bool).tril().numpy()
    _check_sdpa(q, k, v, "causal", 0, 1, 0, causal)
    # window >= N and last_q >= N both reduce the triangle to causal
    _check_sdpa(q, k, v, "triangle", 0, N, 0, causal)
    _check_sdpa(q, k, v, "triangle", 5, 3, N, causal)


def test_window_or_last_q_covering_everything_is_causal_exactly():
    N = 97
    q, k, v = _rand_qkv(12, 1, 2, 1, N, 8)
    oc, lc = oatt.attention(q, k, v, "causal")
    for args in [(0, N, 0), (7, N + 5, 0), (3, 2, N), (0, 1, N + 1)]:
        o, l = oatt.attention(q, k, v, "triangle", *args)
        assert np.array_equal(o, oc) and np.array_equal(l, lc), args


def test_sliding_window_matches_library_attention():
    N, W = 120, 17
    q, k, v = _rand_qkv(13, 1, 4, 1, N, 8, scale_q=2.0)
    band = torch.ones(N, N, dtype=torch.bool).tril().triu(-(W - 1)).numpy()
    _check_sdpa(q, k, v, "triangle", 0, W, 0, band)


def test_sink_only_matches_library_attention():
    N, S = 80, 6
    q, k, v = _rand_qkv(14, 1, 2, 2, N, 8, scale_q=2.0)
    m = torch.eye(N, dtype=torch.bool)
    m[:, :S] = True
    m = (m & torch.ones(N, N, dtype=torch.bool).tril()).numpy()
    _check_sdpa(q, k, v, "triangle", S, 1, 0, m)


def test_last_rows_only():
    # window 1, no sink: every row before the last block sees only itself,
    # the last `last_q` rows are plain causal rows.
    N, L = 70, 9
    q, k, v = _rand_qkv(15, 1, 3, 1, N, 8)
    o, lse = oatt.attention(q, k, v, "triangle", 0, 1, L)
    oc, lc = oatt.attention(q, k, v, "causal")
    for h in range(3):
        for i in range(N - L):
            assert np.array_equal(o[0, h, i], v[0, 0, i])
            assert abs(lse[0, h, i] - np.dot(q[0, h, i], k[0, 0, i]) / math.sqrt(8)) < 1e-12
    assert np.max(np.abs(o[:, :, N - L:] - oc[:, :, N - L:])) < 1e-13
    assert np.max(np.abs(lse[:, :, N - L:] - lc[:, :, N - L:])) < 1e-13


def test_triangle_rows_equal_causal_rows_where_the_sets_coincide():
    N, W, L = 300, 40, 30
    q, k, v = _rand_qkv(16, 1, 2, 1, N, 8)
    o, lse = oatt.attention(q, k, v, "triangle", 5, W, L)
    oc, lc = oatt.attention(q, k, v, "causal")
    same = np.r_[0:W, N - L:N]
    assert np.max(np.abs(o[:, :, same] - oc[:, :, same])) < 1e-13
    assert np.max(np.abs(lse[:, :, same] - lc[:, :, same])) < 1e-13
    assert np.max(np.abs(o[:, :, W + 10] - oc[:, :, W + 10])) > 1e-3


# ----------------------------------------------------------------- invariants

def test_output_is_convex_combination_of_kept_values():
    N = 160
    q, k, v = _rand_qkv(17, 1, 2, 1, N, 8, scale_q=4.0)
    kw = dict(sink=4, window=20, last_q=10)
    o, _ = oatt.attention(q, k, v, "triangle", **kw)
    for i in range(N):
        keys = omask.kept_keys(i, N, "triangle", **kw)
        lo = v[0, 0, keys].min(axis=0)
        hi = v[0, 0, keys].max(axis=0)
        for h in range(2):
            assert np.all(o[0, h, i] >= lo - 1e-12) and np.all(o[0, h, i] <= hi + 1e-12)


def test_masked_keys_do_not_matter():
    N = 140
    q, k, v = _rand_qkv(18, 1, 2, 1, N, 8)
    kw = dict(sink=5, window=12, last_q=6)
    rng = np.random.default_rng(99)
    for i in (0, 3, 17, 60, 133, 139):
        keys = omask.kept_keys(i, N, "triangle", **kw)
        drop = np.setdiff1d(np.arange(N), keys)
        k2, v2 = k.copy(), v.copy()
        k2[0, 0, drop] = rng.standard_normal((drop.size, 8)) * 100
        v2[0, 0, drop] = rng.standard_normal((drop.size, 8)) * 100
        a = oatt.attention(q, k, v, "triangle", rows=[i], **kw)
        b = oatt.attention(q, k2, v2, "triangle", rows=[i], **kw)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        # and a kept key does matter
        k3 = k.copy()
        k3[0, 0, keys[-1]] += 1.0
        c = oatt.attention(q, k3, v, "triangle", rows=[i], **kw)
        assert not np.array_equal(a[1], c[1])


# ------------------------------------------------------ planted-mistake checks

def test_pins_catch_an_off_by_one_window(monkeypatch):
    real = omask.allowed

    def wrong(i, j, N, kind, sink=0, window=1, last_q=0):
        return real(i, j, N, kind, sink, window + 1, last_q)

    monkeypatch.setattr(omask, "allowed", wrong)
    monkeypatch.setattr(omask, "kept_keys",
                        lambda i, N, kind, sink=0, window=1, last_q=0:
                        np.nonzero(wrong(i, np.arange(N), N, kind, sink, window, last_q))[0])
    with pytest.raises(AssertionError):
        test_sliding_window_matches_library_attention()
    with pytest.raises(AssertionError):
        test_zero_queries_give_uniform_weights(64, 4, 8, 8)


def test_pins_catch_a_wrong_kv_head_mapping(monkeypatch):
    def wrong(q, k, v, kind, sink=0, window=1, last_q=0, scale=None, rows=None, row_block=64):
        # head h reading KV head h % Hkv instead of h // G
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        idx = np.arange(Hq) % Hkv
        return real(q, np.repeat(k[:, idx], 1, axis=1)[:, :Hq], np.repeat(v[:, idx], 1, axis=1)[:, :Hq],
                    kind, sink, window, last_q, scale, rows, row_block)

    real = oatt.attention
    monkeypatch.setattr(oatt, "attention", wrong)
    with pytest.raises(AssertionError):
        test_causal_matches_library_attention()


def test_pins_catch_a_missing_lse_scale(monkeypatch):
    real = oatt.attention

    def wrong(*a, **kw):
        o, lse = real(*a, **kw)
        return o, lse * math.sqrt(a[0].shape[-1])

    monkeypatch.setattr(oatt, "attention", wrong)
    with pytest.raises(AssertionError):
        test_single_token_and_first_row()
