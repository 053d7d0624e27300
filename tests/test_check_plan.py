"""Host plan check (tri_attn_check_plan): every plan the planners produce
passes, and each kind of malformed plan a caller could hand the kernel is
rejected with a message naming the bad entry (the kernel walks the arrays as
given)."""
import numpy as np
import pytest

import static_triangle_sparse_amd as tsa


def _plan(N, kind="triangle", sink=0, window=1, last_q=0, bq=128, bk=64):
    mp = tsa.mask_params(N, kind, sink, window, last_q, bq, bk)
    return (mp,) + tsa.tri_attn_plan(mp)


@pytest.mark.parametrize("N,kind,sink,window,last_q,bq,bk", [
    (512, "triangle", 64, 128, 64, 128, 64),
    (1000, "triangle", 5, 70, 33, 128, 64),
    (300, "triangle", 0, 1, 0, 16, 32),
    (257, "causal", 0, 1, 0, 32, 16),
    (32768, "triangle", 128, 2048, 128, 128, 64),
    (131072, "triangle", 128, 2048, 128, 128, 64),
    (1, "triangle", 0, 1, 0, 128, 64),
])
def test_planner_output_passes(N, kind, sink, window, last_q, bq, bk):
    mp, rp, kt, fl = _plan(N, kind, sink, window, last_q, bq, bk)
    tsa.tri_attn_check_plan(mp, rp, kt, fl)


def test_per_head_plan_passes_and_a_wrong_head_fails():
    sink, window = [0, 128, 5], [512, 100, 2048]
    mp = tsa.mask_params(3000, "triangle", 0, 1, 64)
    rp, kt, fl = tsa.tri_attn_plan_heads(mp, sink, window)
    tsa.tri_attn_check_plan(mp, rp, kt, fl, sink, window)
    with pytest.raises(tsa.TriAttnError, match="holds no kept pair|flagged"):
        tsa.tri_attn_check_plan(mp, rp, kt, fl, sink[::-1], window[::-1])


def test_dynamic_subset_of_the_causal_plan_passes():
    # a selection that keeps some tiles of each causal row (and the tiles on
    # the diagonal) with causal flags
    N = 1500
    mp, rp, kt, fl = _plan(N, "causal")
    rng = np.random.default_rng(3)
    keep = rng.random(kt.size) < 0.5
    keep |= fl == tsa.TRI_TILE_PARTIAL
    rows = np.repeat(np.arange(rp.size - 1), np.diff(rp))
    rp2 = np.concatenate([[0], np.cumsum(np.bincount(rows[keep], minlength=rp.size - 1))])
    tsa.tri_attn_check_plan(mp, rp2, kt[keep], fl[keep])
    # the same lists repeated for 3 (batch, head) rows
    nq = rp.size - 1
    rp3 = np.concatenate([[0], np.cumsum(np.tile(np.diff(rp2), 3))])
    tsa.tri_attn_check_plan(mp, rp3, np.tile(kt[keep], 3), np.tile(fl[keep], 3))
    assert rp3.size - 1 == 3 * nq


def _corrupt(which):
    mp, rp, kt, fl = _plan(4096, "triangle", 128, 512, 128)
    rp, kt, fl = rp.copy(), kt.copy(), fl.copy()
    t = 20
    e = rp[t]
    if which == "negative tile":
        kt[e] = -1
    elif which == "tile past the row":
        kt[rp[t + 1] - 1] = 4096 // 64 + 3
    elif which == "not ascending":
        kt[e], kt[e + 1] = kt[e + 1], kt[e]
    elif which == "row_ptr decreasing":
        rp[t + 1] = rp[t] - 1
    elif which == "row_ptr past nnz":
        rp[t + 1] = kt.size + 5
    elif which == "row_ptr[0]":
        rp[0] = 1
    elif which == "last row_ptr":
        rp[-1] -= 1
    elif which == "FULL flag on a partial tile":
        fl[rp[t + 1] - 1] = tsa.TRI_TILE_FULL
    elif which == "PARTIAL flag on a full tile":
        fl[e] = tsa.TRI_TILE_PARTIAL
    elif which == "skipped tile listed":
        # a middle tile of query tile 20 (outside sink and window) replaces a kept one
        row = dict(zip(kt[e:rp[t + 1]].tolist(), fl[e:rp[t + 1]].tolist()))
        mid = 10
        assert mid not in row
        kt[e + 2] = mid
        kt[e:rp[t + 1]] = np.sort(kt[e:rp[t + 1]])
        fl[e:rp[t + 1]] = [row.get(int(x), tsa.TRI_TILE_PARTIAL) for x in kt[e:rp[t + 1]]]
    return mp, rp, kt, fl


CORRUPTIONS = ["negative tile", "tile past the row", "not ascending", "row_ptr decreasing",
               "row_ptr past nnz", "row_ptr[0]", "last row_ptr", "FULL flag on a partial tile",
               "PARTIAL flag on a full tile", "skipped tile listed"]


@pytest.mark.parametrize("which", CORRUPTIONS)
def test_malformed_plans_are_rejected(which):
    mp, rp, kt, fl = _corrupt(which)
    with pytest.raises(tsa.TriAttnError) as e:
        tsa.tri_attn_check_plan(mp, rp, kt, fl)
    assert e.value.status == tsa.TRI_ERR_INVALID
    assert "row" in str(e.value) or "row_ptr" in str(e.value)


def test_argument_errors():
    mp, rp, kt, fl = _plan(512, "triangle", 64, 128, 64)
    with pytest.raises(tsa.TriAttnError, match="multiple"):
        tsa.tri_attn_check_plan(mp, rp[:-1], kt[:rp[-2]], fl[:rp[-2]])
    with pytest.raises(ValueError):
        tsa.tri_attn_check_plan(mp, rp, kt, fl[:-1])
    with pytest.raises(tsa.TriAttnError, match="triangle mask"):
        tsa.tri_attn_check_plan(tsa.mask_params(512, "causal"), rp, kt, fl, [0], [1])
