"""Static mask of a TriangleMix layer and the kept-tile list it induces.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings of the pages (TriangleMix blog "介绍"; 36kr interview, technical
motivation).  The pages give no formula and the triangle figure is missing,
so the plainest reading consistent with the region names is taken:

* keys are token positions 0..N-1, queries likewise (square prefill, no KV
  offset); everything is intersected with causality ``j <= i``;
* the streaming region = the first ``sink`` keys for every query, plus a
  sliding window of ``window`` keys ending at the diagonal (``i - j < window``,
  so the diagonal itself counts towards the window);
* the "Last Q-K" (final aggregation) region = the last ``last_q`` query rows
  (``i >= N - last_q``), which attend to every earlier key;
* everything else ("Middle Q-K") is skipped;
* a dense (shallow) layer keeps the full causal set.

Tile lists use the same grid the GPU kernel walks: query tile ``t`` covers
rows [t*Bq, min(N, (t+1)*Bq)), key tile ``kt`` covers columns
[kt*Bk, (kt+1)*Bk).  A key tile is kept for a query tile if any allowed
(row, column) pair falls in it; a kept tile is FULL if every valid row of the
query tile allows every nominal column of the key tile (columns >= N are never
allowed), and PARTIAL otherwise.  Kept tiles are listed in ascending order.
"""
from __future__ import annotations

import numpy as np

TRIANGLE = "triangle"
CAUSAL = "causal"

FULL = 0
PARTIAL = 1


def allowed(i, j, N, kind, sink=0, window=1, last_q=0):
    """Boolean mask predicate, broadcasting over integer arrays ``i`` (query
    positions) and ``j`` (key positions)."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    causal = (j >= 0) & (j <= i) & (j < N)
    if kind == CAUSAL:
        return causal
    if kind != TRIANGLE:
        raise ValueError(f"unknown mask kind {kind!r}")
    in_sink = j < sink
    in_window = (i - j) < window
    in_last_q = i >= (N - last_q)
    return causal & (in_sink | in_window | in_last_q)


def kept_keys(i, N, kind, sink=0, window=1, last_q=0):
    """Sorted key positions that query row ``i`` attends to, built as the
    union of the three regions (sink, window, last-Q), each straight from its
    definition.  ``allowed`` is the element-level statement of the same set;
    tests check the two agree."""
    i = int(i)
    if kind == CAUSAL or i >= N - last_q:
        return np.arange(0, i + 1, dtype=np.int64)
    sink_part = np.arange(0, min(sink, i + 1), dtype=np.int64)
    win_part = np.arange(max(0, i - window + 1), i + 1, dtype=np.int64)
    return np.union1d(sink_part, win_part)


def dense_mask(N, kind, sink=0, window=1, last_q=0):
    """The full N x N boolean mask (small N only)."""
    r = np.arange(N)
    return allowed(r[:, None], r[None, :], N, kind, sink, window, last_q)


def brute_tiles(N, block_q, block_k, kind, sink=0, window=1, last_q=0):
    """Kept-tile list by brute force over the N x N mask (small N only).

    Returns ``(row_ptr int32[nq+1], k_tile int32[nnz], flags uint8[nnz])``.
    """
    nq = -(-N // block_q)
    nk = -(-N // block_k)
    m = dense_mask(N, kind, sink, window, last_q)
    padded = np.zeros((N, nk * block_k), dtype=bool)
    padded[:, :N] = m
    row_ptr = [0]
    k_tile = []
    flags = []
    for t in range(nq):
        rows = padded[t * block_q: min(N, (t + 1) * block_q)]
        tiles = rows.reshape(rows.shape[0], nk, block_k)
        any_ = tiles.any(axis=(0, 2))
        all_ = tiles.all(axis=(0, 2))
        for kt in range(nk):
            if any_[kt]:
                k_tile.append(kt)
                flags.append(FULL if all_[kt] else PARTIAL)
        row_ptr.append(len(k_tile))
    return (np.asarray(row_ptr, dtype=np.int32), np.asarray(k_tile, dtype=np.int32),
            np.asarray(flags, dtype=np.uint8))


def interval_tiles(N, block_q, block_k, kind, sink=0, window=1, last_q=0):
    """Kept-tile list from per-row key intervals, for sizes where the N x N
    mask does not fit (used at the full benchmark sizes).

    Each row's kept set is at most two intervals: [0, a) (sink) and [b, i]
    (window), or the single interval [0, i] (last-Q rows, causal mode).  A key
    tile [c0, c1] meets a row if it meets either interval; the row covers the
    tile if c1 < N and the tile lies inside one interval, or inside their
    union when the two intervals touch.
    """
    nq = -(-N // block_q)
    nk = -(-N // block_k)
    c0 = np.arange(nk, dtype=np.int64) * block_k
    c1 = c0 + block_k - 1
    row_ptr = [0]
    k_parts = []
    f_parts = []
    for t in range(nq):
        i = np.arange(t * block_q, min(N, (t + 1) * block_q), dtype=np.int64)[:, None]
        if kind == CAUSAL:
            full_row = np.ones_like(i, dtype=bool)
        else:
            full_row = i >= N - last_q
        # interval A = [0, a_hi], interval B = [b_lo, i]; empty A has a_hi = -1
        a_hi = np.where(full_row, i, np.minimum(sink, i + 1) - 1)
        b_lo = np.where(full_row, 0, np.maximum(0, i - window + 1))
        meets_a = (a_hi >= 0) & (c0[None, :] <= a_hi)
        meets_b = (c0[None, :] <= i) & (c1[None, :] >= b_lo)
        any_ = (meets_a | meets_b).any(axis=0)
        inside_a = c1[None, :] <= a_hi
        inside_b = (c0[None, :] >= b_lo) & (c1[None, :] <= i)
        joined = b_lo <= a_hi + 1
        inside_ab = joined & (c1[None, :] <= i)
        covers = (c1[None, :] < N) & (inside_a | inside_b | inside_ab)
        all_ = covers.all(axis=0)
        kts = np.nonzero(any_)[0]
        k_parts.append(kts.astype(np.int32))
        f_parts.append(np.where(all_[kts], FULL, PARTIAL).astype(np.uint8))
        row_ptr.append(row_ptr[-1] + kts.size)
    return (np.asarray(row_ptr, dtype=np.int32),
            np.concatenate(k_parts) if k_parts else np.zeros(0, np.int32),
            np.concatenate(f_parts) if f_parts else np.zeros(0, np.uint8))
