"""Dynamic block-sparse tile selection for the dense (shallow) layers, and
attention over an explicit per-head tile list.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the FlashPrefill page.  Section 2.1 finds the important key blocks
with evenly spread query rows used as probes, against key blocks replaced by
the average of their key vectors; the score computation and the pooling are
one fused pass.  Section 2.2 keeps, for each query block, every key block
whose score reaches alpha times the largest score of that query block (no
sort, no cumulative sum).  Section 2.3 walks only the kept blocks through an
index list.  The TriangleMix pages say the shallow (dense) layers may use such
a dynamic sparse method on top of the static triangle layers.

The pages leave the details open; the readings taken here (the same ones the
GPU library implements) are:

* blocks are the attention kernel's tiles: query tile t = rows
  [t*Bq, min(N, (t+1)*Bq)), key tile kt = keys [kt*Bk, min(N, (kt+1)*Bk));
* the pooled key of a tile is the mean of its keys (keys >= N excluded),
  rounded to bfloat16 -- the precision the GPU scores it in, so that both
  sides take the keep decision on the same values;
* the probes of query tile t are the rows t*Bq + p*(Bq/P), p = 0..P-1
  (P = 16), that are < N;
* probe i sees the key tiles that start at or before it (kt*Bk <= i); its
  logits z = scale * <q_i, pooled key>; its attention over the tiles it sees
  is the softmax of z;
* the score of key tile kt for query tile t is that attention, averaged over
  the tile's probes (a probe that does not see kt contributes 0);
* key tile kt (0 <= kt*Bk <= last row of t) is kept when
  score >= alpha * max score, and always when it crosses the causal diagonal
  of the query tile (kt*Bk + Bk - 1 > t*Bq), so every row keeps its own key;
* kept tiles are listed in ascending order with the causal FULL/PARTIAL flag
  (FULL iff every key of the tile is <= the tile's first row);
* attention over a list keeps, for row i, the keys of the listed tiles that
  are <= i.

Everything is float64 from the exact bf16 inputs, except the one rounding
named above.  Pins: tests/test_oracle_dynamic.py.
"""
from __future__ import annotations

import math

import numpy as np

from . import mask as _mask

N_PROBE = 16


def _round_bf16(x):
    """float64 -> float32 (nearest) -> bfloat16 (nearest, ties to even),
    returned as float64.  Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pooled_keys(k, block_k=64, to_bf16=True):
    """Mean key of every key tile: k [B, Hkv, N, d] -> [B, Hkv, nk, d]."""
    k = np.asarray(k, dtype=np.float64)
    B, H, N, d = k.shape
    nk = -(-N // block_k)
    out = np.zeros((B, H, nk, d), dtype=np.float64)
    for kt in range(nk):
        c0, c1 = kt * block_k, min(N, (kt + 1) * block_k)
        out[:, :, kt] = k[:, :, c0:c1].sum(axis=2) / (c1 - c0)
    return _round_bf16(out) if to_bf16 else out


def probe_rows(t, N, block_q=128, n_probe=N_PROBE):
    """Probe query rows of query tile t (the evenly spaced rows that are < N)."""
    step = block_q // n_probe
    r = t * block_q + step * np.arange(n_probe, dtype=np.int64)
    return r[r < N]


def tile_scores(q_rows, kbar, rows, last_row, scale, block_k=64):
    """Scores of the key tiles 0..last_row//block_k for one query tile.

    q_rows [P, d]: the probe queries (float64); kbar [nk, d]: pooled keys of
    the query's KV head; rows: the probes' positions.  Returns float64
    [last_row//block_k + 1].
    """
    n_cand = last_row // block_k + 1
    z = scale * (np.asarray(q_rows, np.float64) @ kbar[:n_cand].T)          # [P, n_cand]
    sees = (np.arange(n_cand)[None, :] * block_k) <= np.asarray(rows)[:, None]
    z = np.where(sees, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


def select_tiles(q, k, alpha, scale=None, block_q=128, block_k=64, n_probe=N_PROBE,
                 return_scores=False, pooled_bf16=True):
    """Per-(batch, head) kept-tile lists of a dense layer.

    q [B, Hq, N, d], k [B, Hkv, N, d].  Returns CSR over rows
    r = (b * Hq + h) * nq + t: ``(row_ptr int64[B*Hq*nq + 1], k_tile int32,
    flags uint8)``; with ``return_scores`` also a list (indexed by r) of
    (scores, threshold) pairs.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kbar = pooled_keys(k, block_k, to_bf16=pooled_bf16)
    nq = -(-N // block_q)
    row_ptr = [0]
    k_tile, flags, scores = [], [], []
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in range(nq):
                last_row = min(N, (t + 1) * block_q) - 1
                rows = probe_rows(t, N, block_q, n_probe)
                s = tile_scores(q[b, h, rows], kbar[b, g], rows, last_row, scale, block_k)
                thr = alpha * s.max()
                kts = np.arange(s.size)
                diag = kts * block_k + block_k - 1 > t * block_q
                keep = (s >= thr) | diag
                sel = kts[keep]
                k_tile.append(sel.astype(np.int32))
                flags.append(np.where(diag[keep], _mask.PARTIAL, _mask.FULL).astype(np.uint8))
                row_ptr.append(row_ptr[-1] + sel.size)
                scores.append((s, thr))
    out = (np.asarray(row_ptr, dtype=np.int64),
           np.concatenate(k_tile) if k_tile else np.zeros(0, np.int32),
           np.concatenate(flags) if flags else np.zeros(0, np.uint8))
    return out + (scores,) if return_scores else out


def attention_tiles(q, k, v, row_ptr, k_tile, heads=None, scale=None, block_q=128, block_k=64,
                    qtiles=None):
    """Attention over explicit per-(batch, head) tile lists (CSR as returned
    by ``select_tiles``): row i of query tile t keeps the keys of its listed
    key tiles that are <= i.

    ``heads``: optional list of (b, h) pairs to compute; ``qtiles``: optional
    list of query tiles.  Returns dicts {(b, h): (o [R, d], lse [R])} over the
    rows of the requested query tiles, in order.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nq = -(-N // block_q)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else heads
    qtiles = range(nq) if qtiles is None else qtiles
    out = {}
    for b, h in heads:
        g = h // G
        os_, ls_ = [], []
        for t in qtiles:
            r = (b * Hq + h) * nq + t
            kts = np.asarray(k_tile[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
            keys = (kts[:, None] * block_k + np.arange(block_k)[None, :]).ravel()
            keys = keys[keys < N]
            rows = np.arange(t * block_q, min(N, (t + 1) * block_q))
            z = scale * (q[b, h, rows] @ np.asarray(k[b, g, keys], np.float64).T)
            z = np.where(keys[None, :] <= rows[:, None], z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            p = np.exp(z - m)
            l = p.sum(axis=1, keepdims=True)
            os_.append(p @ np.asarray(v[b, g, keys], np.float64) / l)
            ls_.append((m + np.log(l))[:, 0])
        out[(b, h)] = (np.concatenate(os_), np.concatenate(ls_))
    return out
