"""Shared helpers of the GPU parity tests: seeded inputs on host and device,
a call through the C ABI, and the parity bar against the oracle.

Parity bar (per the target of this kernel): output max-abs error <= 1e-2
against the float64 oracle when O is stored in f32; when O is stored in bf16
the rounding of the store itself is allowed on top (half a bf16 ulp of the
reference value); per-row LSE error |dlse| / max(1, |lse|) <= 1e-3 (the floor
keeps rows whose lse is near 0 -- e.g. row 0, where lse = z_00 -- from
turning a 1e-7 absolute error into a large relative one).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import static_triangle_sparse_amd as tsa
import synth
from oracle import attention as oatt

O_ABS_TOL = 1e-2
LSE_REL_TOL = 1e-3


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    tsa.load()  # raises if the library is missing: no fallback path
    return torch.device("cuda:0")


def bits_to_device(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def make_inputs(seed, B, Hq, Hkv, N, d, dev):
    qb, kb, vb = synth.qkv_bf16_bits(seed, B, Hq, Hkv, N, d)
    return (qb, kb, vb), tuple(bits_to_device(x, dev) for x in (qb, kb, vb))


def as_f64(bits):
    return synth.bf16_bits_to_f64(bits)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def run(q, k, v, mode, sink=0, window=1, last_q=0, o_dtype=torch.float32, scale=None):
    """One layer through the C ABI; outputs start as NaN so an unwritten row
    cannot pass."""
    B, Hq, N, d = q.shape
    out = torch.full((B, Hq, N, d), float("nan"), dtype=o_dtype, device=q.device)
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    o, lse = tsa.prefill(q, k, v, mode=mode, sink=sink, window=window, last_q=last_q,
                         o_dtype=o_dtype, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def check(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Compare GPU rows against oracle rows (same shapes)."""
    o = o_gpu.float().cpu().numpy().astype(np.float64) if isinstance(o_gpu, torch.Tensor) else o_gpu
    lse = lse_gpu.cpu().numpy().astype(np.float64) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    bf16 = isinstance(o_gpu, torch.Tensor) and o_gpu.dtype == torch.bfloat16
    tol = O_ABS_TOL + (bf16_half_ulp(o_ref) if bf16 else 0.0)
    err = np.abs(o - o_ref)
    worst = float(np.max(err - tol)) if err.size else -1.0
    assert worst <= 0.0, f"{what}: O error {float(np.max(err)):.3e} exceeds bound (margin {worst:.3e})"
    rel = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    assert float(np.max(rel, initial=0.0)) <= LSE_REL_TOL, f"{what}: LSE rel error {float(np.max(rel)):.3e}"
    return float(np.max(err, initial=0.0)), float(np.max(rel, initial=0.0))


def oracle(bits, mode, sink=0, window=1, last_q=0, rows=None, scale=None):
    qb, kb, vb = bits
    return oatt.attention(as_f64(qb), as_f64(kb), as_f64(vb), mode, sink, window, last_q,
                          scale=scale, rows=rows)


def sample_rows(N, seed=0, extra_tiles=()):
    """Rows of query tiles {0, 1, 15, 16, 17, 8 seeded-random middle tiles,
    nq-2, nq-1} (tiles 15..17 straddle a 2048-token window edge)."""
    nq = -(-N // 128)
    rng = np.random.default_rng(seed)
    tiles = {0, 1, 15, 16, 17, nq - 2, nq - 1, *extra_tiles}
    if nq > 20:
        tiles |= set(int(x) for x in rng.choice(np.arange(18, nq - 2), size=8, replace=False))
    tiles = sorted(t for t in tiles if 0 <= t < nq)
    rows = np.concatenate([np.arange(t * 128, min(N, (t + 1) * 128)) for t in tiles])
    return rows


def oracle_every_row(bits, mode, kw, o_host, lse_host, chunk=512, what=""):
    """Check every query row of a layer against the oracle: rows in chunks,
    each chunk's oracle computed on a worker thread with single-threaded BLAS
    (the products per 64-row block are small, so threads over chunks use the
    host cores better than one multi-threaded product at a time).
    o_host / lse_host: the GPU outputs copied to host (torch CPU tensors).
    Returns (max |dO|, max rel dLSE) over all rows."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    qb, kb, vb = bits
    qf, kf, vf = as_f64(qb), as_f64(kb), as_f64(vb)
    N = qf.shape[2]
    chunks = [np.arange(s, min(N, s + chunk)) for s in range(0, N, chunk)]

    def one(rows):
        ro, rl = oatt.attention(qf, kf, vf, mode, kw.get("sink", 0), kw.get("window", 1),
                                kw.get("last_q", 0), rows=rows)
        sl = slice(int(rows[0]), int(rows[-1]) + 1)
        return check(o_host[:, :, sl], lse_host[:, :, sl], ro, rl, f"{what} rows {sl.start}..{sl.stop - 1}")

    workers = max(1, min(16, os.cpu_count() or 1))
    err = rel = 0.0
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for i, (e, r) in enumerate(ex.map(one, chunks)):
            err, rel = max(err, e), max(rel, r)
            if (i + 1) % 32 == 0 or i + 1 == len(chunks):
                note(f"  {what}: {min(N, (i + 1) * chunk)}/{N} rows checked, max|dO|={err:.2e} "
                     f"max rel dLSE={rel:.2e}")
    return err, rel
