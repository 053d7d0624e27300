"""Masked softmax attention in float64: the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The triangle pattern removes key positions from each query's softmax; it does
not approximate anything that remains (TriangleMix blog, "介绍": a static
pattern computed exactly; 36kr interview: the middle Q-K blocks are dropped).
So the oracle is ordinary attention over each row's kept key set K_i:

    g      = h // G                       (G = Hq / Hkv consecutive query heads
                                           share one KV head)
    z_ij   = scale * sum_c q[b,h,i,c] * k[b,g,j,c]          for j in K_i
    m_i    = max_j z_ij
    l_i    = sum_j exp(z_ij - m_i)
    o[b,h,i,:] = sum_j exp(z_ij - m_i) / l_i * v[b,g,j,:]
    lse[b,h,i] = m_i + ln l_i

with scale = 1/sqrt(d) unless given.  Rows are processed in blocks: the keys
of a block are the union of its rows' kept sets (``mask.kept_keys``); the
scores of the block are one BLAS product over those gathered keys, and the
element predicate ``mask.allowed`` removes pairs a row does not keep.
"""
from __future__ import annotations

import math

import numpy as np

from . import mask as _mask


def attention(q, k, v, kind, sink=0, window=1, last_q=0, scale=None, rows=None,
              row_block=64):
    """Oracle attention.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (any real dtype; computed in
    float64).  ``rows``: optional sorted 1-D array of query rows to compute
    (default all N).  Returns ``(o [B, Hq, R, d] float64, lse [B, Hq, R]
    float64)`` for the R requested rows.
    """
    B, Hq, N, d = q.shape
    Bk_, Hkv, Nk, dk = k.shape
    if (Bk_, Nk, dk) != (B, N, d) or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    if Hq % Hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    R = rows.size
    o = np.zeros((B, Hq, R, d), dtype=np.float64)
    lse = np.zeros((B, Hq, R), dtype=np.float64)
    for s in range(0, R, row_block):
        rb = rows[s:s + row_block]
        keys = np.unique(np.concatenate(
            [_mask.kept_keys(i, N, kind, sink, window, last_q) for i in rb]))
        keep = _mask.allowed(rb[:, None], keys[None, :], N, kind, sink, window, last_q)
        for b in range(B):
            for g in range(Hkv):
                ks = np.asarray(k[b, g, keys], dtype=np.float64)          # [K, d]
                vs = np.asarray(v[b, g, keys], dtype=np.float64)          # [K, d]
                qs = np.asarray(q[b, g * G:(g + 1) * G][:, rb], dtype=np.float64)
                z = scale * (qs.reshape(-1, d) @ ks.T)                    # [G*r, K]
                z = z.reshape(G, rb.size, keys.size)
                z = np.where(keep[None], z, -np.inf)
                m = z.max(axis=2, keepdims=True)
                p = np.exp(z - m)
                l = p.sum(axis=2, keepdims=True)
                out = (p.reshape(-1, keys.size) @ vs).reshape(G, rb.size, d) / l
                o[b, g * G:(g + 1) * G, s:s + rb.size] = out
                lse[b, g * G:(g + 1) * G, s:s + rb.size] = (m + np.log(l))[..., 0]
    return o, lse
