"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic. It only draws random numbers and
rounds them to bfloat16, so that both sides of every parity check read the
same exact bf16 values:

* ``qkv_bf16_bits`` draws Q, then K, then V, i.i.d. N(0, 1) in float32 from
  one numpy PCG64 generator seeded with ``seed``, and rounds each value to
  bfloat16 with round-to-nearest-even.  The result is returned as uint16 bit
  patterns (the upper half of the float32 encoding).
* ``bf16_bits_to_f32`` / ``bf16_bits_to_f64`` widen those bit patterns
  exactly.

Layouts are [B, H, N, d] (batch, head, token, channel), d contiguous.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "normal_bf16_bits",
    "qkv_bf16_bits",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Inputs must be finite (the generators below only produce finite values).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16_bits(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) float32 draws of ``shape`` rounded to bf16 bit patterns.

    Drawn in chunks so that very large tensors need only one float32 chunk of
    temporary memory; the values are the same as one ``standard_normal`` call.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tmp = rng.standard_normal(size=e - s, dtype=np.float32)
        out[s:e] = f32_to_bf16_bits(tmp)
    return out.reshape(shape)


def qkv_bf16_bits(seed: int, batch: int, heads_q: int, heads_kv: int, seqlen: int,
                  head_dim: int):
    """Q [B,Hq,N,d], K [B,Hkv,N,d], V [B,Hkv,N,d] as bf16 bit patterns.

    One PCG64 generator per call (per layer in a layer stack: seed = base +
    layer index); Q is drawn first, then K, then V.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = normal_bf16_bits(rng, (batch, heads_q, seqlen, head_dim))
    k = normal_bf16_bits(rng, (batch, heads_kv, seqlen, head_dim))
    v = normal_bf16_bits(rng, (batch, heads_kv, seqlen, head_dim))
    return q, k, v
