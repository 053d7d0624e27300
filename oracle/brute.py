"""Pure-Python brute force of the same attention, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written independently of ``oracle.attention``: scalar loops over every
(batch, head, query, key), the mask tested key by key with plain
comparisons, and sums taken with ``math.fsum`` (exactly rounded).  Used only
to check the vectorised oracle on N <= 64, d <= 8.
"""
from __future__ import annotations

import math


def _keeps(i, j, N, kind, sink, window, last_q):
    if j > i:
        return False
    if kind == "causal":
        return True
    if i >= N - last_q:          # final-aggregation rows see every earlier key
        return True
    if j < sink:                 # leading sink keys
        return True
    return i - j < window        # diagonal window, diagonal included


def attention(q, k, v, kind, sink=0, window=1, last_q=0, scale=None):
    """q, k, v: nested lists or arrays [B][H][N][d].  Returns (o, lse) as
    nested lists [B][Hq][N][d] and [B][Hq][N]."""
    B = len(q)
    Hq = len(q[0])
    N = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = [[[[0.0] * d for _ in range(N)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(N):
                js = [j for j in range(N) if _keeps(i, j, N, kind, sink, window, last_q)]
                z = []
                for j in js:
                    z.append(scale * math.fsum(float(q[b][h][i][c]) * float(k[b][g][j][c])
                                               for c in range(d)))
                m = max(z)
                w = [math.exp(x - m) for x in z]
                l = math.fsum(w)
                for c in range(d):
                    o[b][h][i][c] = math.fsum(w[t] * float(v[b][g][js[t]][c])
                                              for t in range(len(js))) / l
                lse[b][h][i] = m + math.log(l)
    return o, lse
