"""Precision tiers for the triangle layer: far tiles scored with fp8 or fp4 Q and K.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the TriAttention page.  It assigns each query-key tile to skipping,
a lower-precision or a higher-precision score computation, chooses the
regions per head with two diagonal-distance boundaries, and combines the
contributions of both precisions into one normalised attention output.  On
MI355X the native lower-precision matrix format is fp8 (e4m3); the layer's
skipping is the triangle plan itself, so one per-head boundary remains:

* a kept key tile kt of query tile t is LOW precision when its smallest
  query-key distance, t*Bq - (kt*Bk + Bk - 1), is >= dist[h]; otherwise it
  is computed in bf16 as in the plain triangle layer;
* on LOW tiles the score is scale * s_q * s_k * <q8, k8>, with
    - s_q = amax(|q row|) / 448 and q8 = e4m3(q * (448 / amax)),
    - s_k = amax(|K of the key tile|) / 448 and k8 = e4m3(k * (448 / amax)):
      the page assigns a precision to each query-key tile, so the key tile
      (the grid's Bk keys) is the block that shares one scale,
  every scale and product formed in float32 as the GPU forms them (the
  rounding of a value to a code is an integer decision: both sides take it
  in the same precision); an all-zero row or key tile has scale 0;
* values are then combined in one softmax over the row's kept keys.

The page's tiers are 4-bit and 8-bit; a second per-head boundary dist4 adds
the 4-bit one: a kept tile whose smallest distance is >= dist4[h] is scored
in fp4 (e2m1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), with s_q = amax / 6,
s_k = amax of the key tile / 6 and codes e2m1(clamp(x * 6 / amax)),
rounded to nearest, ties to the even code, in float32 as on the GPU.  The
farthest tier wins: fp4 if d >= dist4, else fp8 if d >= dist, else bf16.

P and V stay bf16 (only the scores change precision); the oracle's softmax
and PV are float64.  Pins: tests/test_oracle_tiers.py.
"""
from __future__ import annotations

import math

import numpy as np

from . import mask as _mask

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_values():
    """All 256 e4m3 codes decoded (NaN for the two NaN codes 0x7F, 0xFF)."""
    out = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * m / 8.0 * 2.0 ** -6
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def round_e4m3(x):
    """Round float32 values to e4m3 (nearest, ties to even), saturating at
    +-448.  Returns float64 values of the chosen codes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade (normal: 2^-6 .. 2^8); below 2^-6 the subnormal
    # step 2^-9 applies
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3)
    q = a / step
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    v = (r + up) * step
    return np.copysign(np.minimum(v, E4M3_MAX), x)


def e2m1_values():
    """All 16 e2m1 codes decoded: sign bit 3, exponent bits 2-1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0 or 0.5)."""
    out = np.empty(16)
    for c in range(16):
        s = -1.0 if c & 8 else 1.0
        e = (c >> 1) & 3
        m = c & 1
        out[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return out


def round_e2m1(x):
    """Round values to e2m1 (nearest, ties to the even code), saturating at
    +-6.  Returns float64 values of the chosen codes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    # the binade step: 0.5 below 2 (subnormal 0..0.5 and 1..2), 1 on [2, 4), 2 on [4, 6]
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = a / step
    r = np.floor(q)
    frac = q - r
    # the code's mantissa bit is the parity of r within its binade (r even: even code)
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    v = np.minimum((r + up) * step, E2M1_MAX)
    return np.copysign(v, x)


def quantize4(x, axis=None):
    """(codes as float64 values, scale) of a block in fp4: float32 arithmetic
    as on the GPU.  ``axis``: reduce amax over this axis (keepdims)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=axis, keepdims=axis is not None).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E2M1_MAX) / amax, np.float32(0)).astype(np.float32)
    y = (x32 * inv).astype(np.float32)
    scale = (amax / np.float32(E2M1_MAX)).astype(np.float32)
    return round_e2m1(y), scale


def quantize(x, axis=None):
    """(codes as float64 values, scale) of a block: float32 arithmetic as on
    the GPU.  ``axis``: reduce amax over this axis (keepdims)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=axis, keepdims=axis is not None).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
    y = (x32 * inv).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return round_e4m3(y), scale


def low_tile(t, kt, dist, block_q=128, block_k=64):
    """True when the smallest query-key distance of key tile kt of query tile
    t reaches the boundary `dist`."""
    return t * block_q - (kt * block_k + block_k - 1) >= dist


def attention(q, k, v, sink, window, last_q, dist, scale=None, rows=None, block_q=128, block_k=64,
              dist4=None):
    """Triangle attention with fp8 (and fp4) scores on far tiles.

    q [B, Hq, N, d], k/v [B, Hkv, N, d] (exact bf16 values); dist: per query
    head fp8 boundary, dist4: per query head fp4 boundary (None: no fp4
    tier).  Returns (o [B, Hq, R, d], lse [B, Hq, R]) for the requested rows
    (default all), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, np.int64)
    nk = -(-N // block_k)
    # quantized keys per key tile (keys >= N are zero, as the GPU loads them)
    kp = np.zeros((B, Hkv, nk * block_k, d))
    kp[:, :, :N] = k
    kq, ks = quantize(kp.reshape(B, Hkv, nk, block_k * d), axis=3)
    k8 = kq.reshape(B, Hkv, nk * block_k, d)[:, :, :N]
    s_k = np.repeat(ks[..., 0], block_k, axis=2)[:, :, :N]            # [B, Hkv, N]
    kq4, ks4 = quantize4(kp.reshape(B, Hkv, nk, block_k * d), axis=3)
    k4 = kq4.reshape(B, Hkv, nk * block_k, d)[:, :, :N]
    s_k4 = np.repeat(ks4[..., 0], block_k, axis=2)[:, :, :N]
    o = np.zeros((B, Hq, rows.size, d))
    lse = np.zeros((B, Hq, rows.size))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for n, i in enumerate(rows):
                keys = _mask.kept_keys(i, N, "triangle", sink, window, last_q)
                q8, s_q = quantize(q[b, h, i])
                t = i // block_q
                low = low_tile(t, keys // block_k, dist[h], block_q, block_k)
                z_hi = scale * (k[b, g, keys] @ q[b, h, i])
                acc = k8[b, g, keys] @ q8
                z_lo = scale * (np.float64(s_q) * s_k[b, g, keys]) * acc
                z = np.where(low, z_lo, z_hi)
                if dist4 is not None:
                    q4, s_q4 = quantize4(q[b, h, i])
                    far = low_tile(t, keys // block_k, dist4[h], block_q, block_k)
                    z_4 = scale * (np.float64(s_q4) * s_k4[b, g, keys]) * (k4[b, g, keys] @ q4)
                    z = np.where(far, z_4, z)
                m = z.max()
                p = np.exp(z - m)
                l = p.sum()
                o[b, h, n] = p @ v[b, g, keys] / l
                lse[b, h, n] = m + math.log(l)
    return o, lse
