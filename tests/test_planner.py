"""The C planner (tri_attn_plan, through the C ABI) against the oracle's
brute-force tile enumeration, bit for bit."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import static_triangle_sparse_amd as tsa
from oracle import mask as omask

KINDS = {"triangle": tsa.TRI_MASK_TRIANGLE, "causal": tsa.TRI_MASK_CAUSAL}


def _plan(N, bq, bk, kind, sink, window, last_q):
    return tsa.tri_attn_plan(tsa.mask_params(N, KINDS[kind], sink, window, last_q, bq, bk))


def _same(a, b):
    return all(np.array_equal(np.asarray(x), np.asarray(y)) and np.asarray(x).dtype == np.asarray(y).dtype
               for x, y in zip(a, b))


def test_exhaustive_small_grids():
    n_cases = 0
    for N in list(range(1, 70)) + [127, 128, 129, 200, 255, 256, 257, 300]:
        for bq, bk in [(16, 16), (32, 16), (16, 64), (64, 32), (128, 64), (32, 128)]:
            for kind, sink, window, last_q in [
                ("causal", 0, 1, 0), ("triangle", 0, 1, 0), ("triangle", 1, 1, 1),
                ("triangle", 3, 7, 5), ("triangle", 16, 16, 16), ("triangle", 17, 33, 0),
                ("triangle", 0, 40, 70), ("triangle", 64, 128, 64), ("triangle", 50, 10, 0),
                ("triangle", N + 3, 2, 0), ("triangle", 2, N + 1, 0), ("triangle", 0, 1, N + 9),
            ]:
                got = _plan(N, bq, bk, kind, sink, window, last_q)
                ref = omask.brute_tiles(N, bq, bk, kind, sink, window, last_q)
                assert _same(got, ref), (N, bq, bk, kind, sink, window, last_q)
                n_cases += 1
    assert n_cases > 5000


@settings(max_examples=300, deadline=None)
@given(N=st.integers(1, 400), bq=st.integers(1, 130), bk=st.integers(1, 130),
       causal=st.booleans(), sink=st.integers(0, 500), window=st.integers(1, 500),
       last_q=st.integers(0, 500))
def test_fuzz_against_brute_force(N, bq, bk, causal, sink, window, last_q):
    kind = "causal" if causal else "triangle"
    assert _same(_plan(N, bq, bk, kind, sink, window, last_q),
                 omask.brute_tiles(N, bq, bk, kind, sink, window, last_q))


@pytest.mark.parametrize("N,kind,expect_nnz,expect_partial", [
    (512, "triangle", 19, 15), (512, "causal", 20, 8),
    (32768, "triangle", None, None), (131072, "triangle", None, None), (32768, "causal", None, None),
])
def test_benchmark_sizes_against_interval_enumerator(N, kind, expect_nnz, expect_partial):
    sink, window, last_q = (64, 128, 64) if N == 512 else (128, 2048, 128)
    got = _plan(N, 128, 64, kind, sink, window, last_q)
    ref = omask.interval_tiles(N, 128, 64, kind, sink, window, last_q)
    assert _same(got, ref)
    if expect_nnz is not None:
        assert got[1].size == expect_nnz and int(got[2].sum()) == expect_partial


def test_triangle_equals_causal_when_window_covers_everything():
    for N in (1, 100, 1000, 4097):
        tri = _plan(N, 128, 64, "triangle", 7, N, 0)
        cau = _plan(N, 128, 64, "causal", 0, 1, 0)
        assert _same(tri, cau)


def test_kernel_causal_range_rule():
    # The dense kernel enumerates tiles 0..(r1/64) of query tile t and masks a
    # tile iff its last column passes the first row or the sequence end; that
    # rule must equal the planner's causal list.
    for N in (1, 63, 64, 65, 127, 128, 129, 1000, 4096, 5000):
        row_ptr, k_tile, flags = _plan(N, 128, 64, "causal", 0, 1, 0)
        for t in range(row_ptr.size - 1):
            r0, r1 = t * 128, min(N, (t + 1) * 128) - 1
            kts = np.arange(0, r1 // 64 + 1)
            c1 = kts * 64 + 63
            part = (c1 > r0) | (c1 >= N)
            assert np.array_equal(k_tile[row_ptr[t]:row_ptr[t + 1]], kts)
            assert np.array_equal(flags[row_ptr[t]:row_ptr[t + 1]], part.astype(np.uint8))


def test_empty_sequence():
    row_ptr, k_tile, flags = _plan(0, 128, 64, "triangle", 1, 1, 1)
    assert row_ptr.tolist() == [0] and k_tile.size == 0 and flags.size == 0


# ------------------------------------------------------ per-head boundaries

@pytest.mark.parametrize("N,bq,bk,last_q", [(300, 32, 16, 20), (1000, 128, 64, 64), (129, 128, 64, 0),
                                            (5000, 128, 64, 128)])
def test_per_head_plan_is_the_brute_force_plan_of_each_head(N, bq, bk, last_q):
    # head h's rows of the per-head CSR are the oracle's tile list for that
    # head's (sink, window) -- TriAttention page: per-head boundaries
    heads = [(0, 1), (4, 100), (200, N + 5), (N + 1, 3), (17, 33), (64, 2048)]
    sink = [s for s, _ in heads]
    window = [w for _, w in heads]
    rp, kt, fl = tsa.tri_attn_plan_heads(tsa.mask_params(N, "triangle", 0, 1, last_q, bq, bk),
                                         sink, window)
    nq = -(-N // bq)
    assert rp.size == len(heads) * nq + 1
    for h, (s, w) in enumerate(heads):
        ref = (omask.brute_tiles(N, bq, bk, "triangle", s, w, last_q) if N <= 1000 else
               omask.interval_tiles(N, bq, bk, "triangle", s, w, last_q))
        seg = slice(rp[h * nq], rp[(h + 1) * nq])
        assert np.array_equal(kt[seg], ref[1]) and np.array_equal(fl[seg], ref[2]), (h, s, w)
        assert np.array_equal(rp[h * nq:(h + 1) * nq + 1] - rp[h * nq], ref[0])


def test_per_head_plan_rejects_bad_arguments():
    import ctypes
    lib = tsa.load()
    mp = tsa.mask_params(500, "triangle", 0, 1, 0)
    A = lambda x: (ctypes.c_int64 * len(x))(*x)
    nq, nnz = ctypes.c_int32(), ctypes.c_int64()
    call = lambda m, H, s, w: lib.tri_attn_plan_heads(ctypes.byref(m), H, s, w, None, None, None, 0,
                                                      ctypes.byref(nq), ctypes.byref(nnz))
    assert call(mp, 2, A([1, 2]), A([3, 4])) == tsa.TRI_OK
    assert call(mp, 0, A([1]), A([3])) == tsa.TRI_ERR_INVALID
    assert call(mp, 2, A([1, -1]), A([3, 4])) == tsa.TRI_ERR_INVALID
    assert call(mp, 2, A([1, 2]), A([3, 0])) == tsa.TRI_ERR_INVALID
    assert call(mp, 1, None, A([3])) == tsa.TRI_ERR_INVALID
    assert call(tsa.mask_params(500, "causal"), 1, A([1]), A([3])) == tsa.TRI_ERR_INVALID
    assert call(mp, 1, A([1 << 40]), A([3])) == tsa.TRI_ERR_UNSUPPORTED
