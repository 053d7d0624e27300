"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, validates every argument before touching HIP, and its block
schedule covers each work item exactly once."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import static_triangle_sparse_amd as tsa
from static_triangle_sparse_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tri_attn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_symbols_are_exported():
    names = _declared_functions()
    assert {"tri_attn_plan", "tri_attn_prefill", "dense_causal_prefill",
            "tri_attn_last_error", "tri_dyn_plan_sizes", "tri_dyn_plan",
            "tri_attn_prefill_lists", "tri_attn_plan_heads", "tri_attn_prefill_heads",
            "tri_attn_quantize_k_sizes", "tri_attn_quantize_k", "tri_attn_prefill_tiered",
            "tri_attn_split_workspace_size", "tri_attn_prefill_split", "tri_attn_split_work_item",
            "tri_attn_quantize_k4_sizes", "tri_attn_quantize_k4"} <= set(names)
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert tsa.tri_attn_abi_version() == 4


# ----------------------------------------------------------- plan validation

def _raw_plan(mp, row_ptr=None, k_tile=None, flags=None, capacity=0, nq=True, nnz=True):
    lib = _abi.load()
    nq_v = ctypes.c_int32(-7)
    nnz_v = ctypes.c_int64(-7)
    st = lib.tri_attn_plan(ctypes.byref(mp) if mp is not None else None, row_ptr, k_tile, flags,
                           capacity, ctypes.byref(nq_v) if nq else None,
                           ctypes.byref(nnz_v) if nnz else None)
    return st, nq_v.value, nnz_v.value


@pytest.mark.parametrize("field,value", [("seqlen", -1), ("block_q", 0), ("block_k", 0),
                                         ("kind", 2), ("reserved", 1), ("sink", -1),
                                         ("window", 0), ("last_q", -1)])
def test_plan_rejects_bad_params(field, value):
    mp = tsa.mask_params(100, "triangle", 1, 2, 3)
    setattr(mp, field, value)
    st, _, _ = _raw_plan(mp)
    assert st == tsa.TRI_ERR_INVALID
    assert tsa.last_error()


def test_plan_null_and_capacity_errors():
    mp = tsa.mask_params(1000, "triangle", 5, 100, 10)
    assert _raw_plan(None)[0] == tsa.TRI_ERR_INVALID
    assert _raw_plan(mp, nq=False)[0] == tsa.TRI_ERR_INVALID
    assert _raw_plan(mp, nnz=False)[0] == tsa.TRI_ERR_INVALID
    st, nq, nnz = _raw_plan(mp)
    assert st == tsa.TRI_OK and nq == 8 and nnz > 0
    rp = (ctypes.c_int32 * (nq + 1))()
    kt = (ctypes.c_int32 * nnz)()
    fl = (ctypes.c_uint8 * nnz)()
    # partially NULL output arrays
    assert _raw_plan(mp, rp, None, fl, nnz)[0] == tsa.TRI_ERR_INVALID
    # too small
    st, nq2, nnz2 = _raw_plan(mp, rp, kt, fl, nnz - 1)
    assert st == tsa.TRI_ERR_CAPACITY and nq2 == nq and nnz2 == nnz
    assert "capacity" in tsa.last_error()
    assert _raw_plan(mp, rp, kt, fl, nnz)[0] == tsa.TRI_OK
    assert tsa.last_error() == ""


# -------------------------------------------------------- prefill validation

def _good_tensors(B=1, Hq=4, Hkv=2, N=256, d=128, o_dtype=tsa.TRI_DTYPE_BF16):
    t = tsa.AttnTensors()
    base = 1 << 20  # fake, suitably aligned device addresses: never dereferenced
    t.q, t.k, t.v, t.o, t.lse = base, base * 2, base * 3, base * 4, base * 5
    t.batch, t.heads_q, t.heads_kv, t.head_dim, t.seqlen = B, Hq, Hkv, d, N
    t.q_stride[:] = [Hq * N * d, N * d, d]
    t.k_stride[:] = [Hkv * N * d, N * d, d]
    t.v_stride[:] = [Hkv * N * d, N * d, d]
    t.o_stride[:] = [Hq * N * d, N * d, d]
    t.lse_stride[:] = [Hq * N, N]
    t.softmax_scale = d ** -0.5
    t.o_dtype = o_dtype
    return t


BAD_TENSORS = [
    ("q", None, tsa.TRI_ERR_INVALID), ("k", None, tsa.TRI_ERR_INVALID),
    ("v", None, tsa.TRI_ERR_INVALID), ("o", None, tsa.TRI_ERR_INVALID),
    ("q", (1 << 20) + 8, tsa.TRI_ERR_INVALID), ("k", (1 << 21) + 2, tsa.TRI_ERR_INVALID),
    ("o", (1 << 22) + 4, tsa.TRI_ERR_INVALID), ("lse", (1 << 22) + 2, tsa.TRI_ERR_INVALID),
    ("batch", 0, tsa.TRI_ERR_INVALID), ("heads_q", 0, tsa.TRI_ERR_INVALID),
    ("heads_kv", 0, tsa.TRI_ERR_INVALID), ("heads_q", 5, tsa.TRI_ERR_INVALID),
    ("head_dim", 96, tsa.TRI_ERR_UNSUPPORTED), ("head_dim", 256, tsa.TRI_ERR_UNSUPPORTED),
    ("seqlen", -1, tsa.TRI_ERR_INVALID), ("seqlen", 1 << 30, tsa.TRI_ERR_UNSUPPORTED),
    ("o_dtype", 7, tsa.TRI_ERR_INVALID), ("softmax_scale", 0.0, tsa.TRI_ERR_INVALID),
    ("softmax_scale", float("inf"), tsa.TRI_ERR_INVALID),
    ("softmax_scale", float("nan"), tsa.TRI_ERR_INVALID),
]


@pytest.mark.parametrize("field,value,status", BAD_TENSORS)
def test_dense_prefill_rejects_bad_tensors(field, value, status):
    t = _good_tensors(o_dtype=tsa.TRI_DTYPE_F32)
    setattr(t, field, value)
    st = _abi.load().dense_causal_prefill(ctypes.byref(t), None)
    assert st == status, tsa.last_error()
    assert tsa.last_error()


def test_prefill_rejects_keys_spanning_2gib():
    t = _good_tensors(N=1 << 16)
    t.k_stride[2] = 1 << 14          # 65536 tokens x 32 KiB = 2 GiB
    assert _abi.load().dense_causal_prefill(ctypes.byref(t), None) == tsa.TRI_ERR_UNSUPPORTED
    t.k_stride[2] = 128
    t.v_stride[2] = 1 << 14
    assert _abi.load().dense_causal_prefill(ctypes.byref(t), None) == tsa.TRI_ERR_UNSUPPORTED


@pytest.mark.parametrize("which,idx,value", [("q_stride", 2, 100), ("k_stride", 1, 4),
                                             ("v_stride", 0, -8), ("o_stride", 2, 2),
                                             ("lse_stride", 0, -1)])
def test_prefill_rejects_bad_strides(which, idx, value):
    t = _good_tensors()
    getattr(t, which)[idx] = value
    assert _abi.load().dense_causal_prefill(ctypes.byref(t), None) == tsa.TRI_ERR_INVALID


def test_triangle_prefill_rejects_bad_plan_arguments():
    lib = _abi.load()
    t = _good_tensors()
    mp = tsa.mask_params(256, "triangle", 4, 64, 16)
    P = 1 << 24
    assert lib.tri_attn_prefill(ctypes.byref(t), None, P, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill(None, ctypes.byref(mp), P, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), None, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), P, None, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), P, P, None, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), P + 2, P, P, None) == tsa.TRI_ERR_INVALID
    bad = tsa.mask_params(256, "triangle", 4, 64, 16, block_q=64)
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(bad), P, P, P, None) == tsa.TRI_ERR_UNSUPPORTED
    bad = tsa.mask_params(255, "triangle", 4, 64, 16)
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(bad), P, P, P, None) == tsa.TRI_ERR_INVALID
    bad = tsa.mask_params(256, "triangle", 4, 0, 16)
    assert lib.tri_attn_prefill(ctypes.byref(t), ctypes.byref(bad), P, P, P, None) == tsa.TRI_ERR_INVALID


def test_empty_sequence_is_a_no_op():
    # N == 0 validates and returns before any HIP call
    t = _good_tensors(N=0)
    assert _abi.load().dense_causal_prefill(ctypes.byref(t), None) == tsa.TRI_OK
    mp = tsa.mask_params(0, "triangle", 4, 64, 16)
    P = 1 << 24
    assert _abi.load().tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), P, P, P, None) == tsa.TRI_OK


# ------------------------------------------------------------ dynamic plan

def _causal_tiles(N):
    return sum((min(N, (t + 1) * 128) - 1) // 64 + 1 for t in range(-(-N // 128)))


def test_dyn_plan_sizes():
    for B, Hq, Hkv, N, d in [(1, 4, 2, 256, 128), (2, 28, 4, 1000, 64), (1, 32, 8, 131072, 128),
                             (1, 1, 1, 1, 64)]:
        t = _good_tensors(B, Hq, Hkv, N, d)
        ws, rows, nnz = tsa.tri_dyn_plan_sizes(t)
        nq, nkt = -(-N // 128), -(-N // 64)
        assert rows == B * Hq * nq
        assert nnz == B * Hq * _causal_tiles(N)
        pooled = -(-(B * Hkv * nkt * d * 2) // 256) * 256
        assert ws >= pooled + B * Hq * nq * (4 * -(-nkt // 32) + 4)
        assert ws % 256 == 0
    assert _causal_tiles(131072) == 1049600  # the dense 128K layer's tile count


def test_dyn_plan_rejects_bad_arguments():
    lib = _abi.load()
    t = _good_tensors(N=1000)
    ws, rows, nnz = tsa.tri_dyn_plan_sizes(t)
    W = 1 << 26  # fake, 256-byte-aligned device addresses: never dereferenced
    P = 1 << 27

    def call(alpha=0.5, n_probe=16, w=W, wbytes=ws, rp=P, kt=P, fl=P, cap=nnz, tt=t):
        dp = tsa.DynParams(alpha, n_probe)
        return lib.tri_dyn_plan(ctypes.byref(tt) if tt is not None else None, ctypes.byref(dp),
                                w, wbytes, rp, kt, fl, cap, None)

    assert call(tt=None) == tsa.TRI_ERR_INVALID
    assert lib.tri_dyn_plan(ctypes.byref(t), None, W, ws, P, P, P, nnz, None) == tsa.TRI_ERR_INVALID
    for a in (-0.1, 1.5, float("nan")):
        assert call(alpha=a) == tsa.TRI_ERR_INVALID
    assert call(n_probe=8) == tsa.TRI_ERR_UNSUPPORTED
    assert call(w=None) == tsa.TRI_ERR_INVALID
    assert call(w=W + 128) == tsa.TRI_ERR_INVALID
    assert call(rp=None) == tsa.TRI_ERR_INVALID
    assert call(kt=P + 2) == tsa.TRI_ERR_INVALID
    assert call(wbytes=ws - 1) == tsa.TRI_ERR_CAPACITY
    assert call(cap=nnz - 1) == tsa.TRI_ERR_CAPACITY
    assert "capacity" in tsa.last_error()
    bad = _good_tensors(N=1000, d=96)
    assert call(tt=bad) == tsa.TRI_ERR_UNSUPPORTED
    # N == 0 validates and returns before any HIP call
    z = _good_tensors(N=0)
    ws0, _, nnz0 = tsa.tri_dyn_plan_sizes(z)
    assert call(tt=z, wbytes=ws0, cap=nnz0) == tsa.TRI_OK


def test_dyn_plan_noalloc_rejects_bad_arguments():
    # every rejection happens before any HIP call (no GPU here)
    lib = _abi.load()
    t = _good_tensors(N=1000)
    ws, rows, nnz = tsa.tri_dyn_plan_sizes(t)
    assert ws <= tsa.TRI_DYN_SCRATCH_BYTES
    P = 1 << 27

    def call(alpha=0.5, n_probe=16, rp=P, kt=P, fl=P, cap=nnz, tt=t):
        dp = tsa.DynParams(alpha, n_probe)
        return lib.tri_dyn_plan_noalloc(ctypes.byref(tt) if tt is not None else None, ctypes.byref(dp),
                                        rp, kt, fl, cap, None)

    assert call(tt=None) == tsa.TRI_ERR_INVALID
    assert call(alpha=2.0) == tsa.TRI_ERR_INVALID
    assert call(n_probe=4) == tsa.TRI_ERR_UNSUPPORTED
    assert call(rp=None) == tsa.TRI_ERR_INVALID
    assert call(kt=P + 2) == tsa.TRI_ERR_INVALID
    assert call(cap=nnz - 1) == tsa.TRI_ERR_CAPACITY
    # a layer whose workspace exceeds the library-owned array
    big = _good_tensors(N=1 << 19, Hq=32, Hkv=8)
    wsb, _, nnzb = tsa.tri_dyn_plan_sizes(big)
    assert wsb > tsa.TRI_DYN_SCRATCH_BYTES
    assert call(tt=big, cap=nnzb) == tsa.TRI_ERR_CAPACITY
    assert "scratch" in tsa.last_error()
    # the largest Llama-shaped layer (batch 1) it holds is N = 337920: the next
    # query tile (N + 128) needs more than the array
    edge = _good_tensors(N=337920, Hq=32, Hkv=8)
    assert tsa.tri_dyn_plan_sizes(edge)[0] <= tsa.TRI_DYN_SCRATCH_BYTES
    past = _good_tensors(N=337920 + 128, Hq=32, Hkv=8)
    assert tsa.tri_dyn_plan_sizes(past)[0] > tsa.TRI_DYN_SCRATCH_BYTES
    assert call(tt=past, cap=tsa.tri_dyn_plan_sizes(past)[2]) == tsa.TRI_ERR_CAPACITY
    z = _good_tensors(N=0)
    assert call(tt=z, cap=tsa.tri_dyn_plan_sizes(z)[2]) == tsa.TRI_OK


def test_prefill_lists_rejects_bad_arguments():
    lib = _abi.load()
    t = _good_tensors()
    P = 1 << 24
    assert lib.tri_attn_prefill_lists(None, P, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_lists(ctypes.byref(t), None, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_lists(ctypes.byref(t), P, None, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_lists(ctypes.byref(t), P, P, None, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_lists(ctypes.byref(t), P + 1, P, P, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_lists(ctypes.byref(_good_tensors(N=0)), P, P, P, None) == tsa.TRI_OK


def test_prefill_heads_rejects_bad_arguments():
    lib = _abi.load()
    t = _good_tensors()
    mp = tsa.mask_params(256, "triangle", 4, 64, 16)
    P = 1 << 24
    args = [P, P, P, P, P]  # a valid call would launch: only the error paths run here
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert lib.tri_attn_prefill_heads(ctypes.byref(t), ctypes.byref(mp), *bad, None) == tsa.TRI_ERR_INVALID
    bad = list(args)
    bad[0] = P + 2
    assert lib.tri_attn_prefill_heads(ctypes.byref(t), ctypes.byref(mp), *bad, None) == tsa.TRI_ERR_INVALID
    causal = tsa.mask_params(256, "causal")
    assert lib.tri_attn_prefill_heads(ctypes.byref(t), ctypes.byref(causal), *args, None) == tsa.TRI_ERR_INVALID
    other = tsa.mask_params(255, "triangle", 4, 64, 16)
    assert lib.tri_attn_prefill_heads(ctypes.byref(t), ctypes.byref(other), *args, None) == tsa.TRI_ERR_INVALID
    z = _good_tensors(N=0)
    mz = tsa.mask_params(0, "triangle", 4, 64, 16)
    assert lib.tri_attn_prefill_heads(ctypes.byref(z), ctypes.byref(mz), *args, None) == tsa.TRI_OK


# ----------------------------------------------------------------- schedule

def _cover(B, Hq, Hkv, N, kind, last_q):
    _, _, _, grid = tsa.tri_attn_work_item(B, Hq, Hkv, N, kind, last_q, 0)
    seen = {}
    order = []
    for bid in range(grid):
        b, h, t, _ = tsa.tri_attn_work_item(B, Hq, Hkv, N, kind, last_q, bid)
        if t < 0:
            continue
        assert (b, h, t) not in seen, (b, h, t)
        seen[(b, h, t)] = bid
        order.append((bid, b, h, t))
    nq = -(-N // 128)
    assert set(seen) == {(b, h, t) for b in range(B) for h in range(Hq) for t in range(nq)}
    assert grid <= B * Hq * (nq + 8)
    return seen, order


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 1, 1, 512), (1, 32, 8, 4096), (1, 28, 4, 3000),
                                        (2, 6, 3, 1000), (3, 7, 7, 129), (1, 4, 1, 1),
                                        (4, 32, 8, 640), (1, 12, 12, 9000)])
@pytest.mark.parametrize("kind", [tsa.TRI_MASK_TRIANGLE, tsa.TRI_MASK_CAUSAL])
def test_schedule_covers_every_item_once(B, Hq, Hkv, N, kind):
    _cover(B, Hq, Hkv, N, kind, 128)


def test_schedule_puts_a_kv_group_on_one_xcd_and_heavy_tiles_first():
    # 8 KV groups: block bid runs on XCD bid % 8, which must own one group
    seen, order = _cover(1, 32, 8, 8192, tsa.TRI_MASK_TRIANGLE, 128)
    for (b, h, t), bid in seen.items():
        assert bid % 8 == h // 4
    nq = 64
    first = [t for bid, b, h, t in order[:32]]
    assert first == [nq - 1] * 32          # the last-Q tile of every head first
    seen, order = _cover(1, 32, 8, 8192, tsa.TRI_MASK_CAUSAL, 0)
    ts = [t for _, _, _, t in order]
    assert ts == sorted(ts, reverse=True)  # causal: heaviest (longest) tiles first


# ----------------------------------------------------------------- split launch

def _cover_split(B, Hq, Hkv, N, last_q, chunk):
    _, _, _, _, grid = tsa.tri_attn_split_work_item(B, Hq, Hkv, N, last_q, chunk, 0)
    nq = -(-N // 128)
    nkt = -(-N // 64)
    first_heavy = (N - min(last_q, N)) // 128 if last_q > 0 else nq
    n_split = -(-nkt // chunk) if first_heavy < nq else 1
    seen = {}
    order = []
    for bid in range(grid):
        b, h, t, c = tsa.tri_attn_split_work_item(B, Hq, Hkv, N, last_q, chunk, bid)[:4]
        if t < 0:
            assert (b, h, c) == (-1, -1, -1)
            continue
        key = (b, h, t, c)
        assert key not in seen, key
        seen[key] = bid
        order.append((bid, b, h, t, c))
    want = set()
    for b in range(B):
        for h in range(Hq):
            for t in range(nq):
                if t >= first_heavy and n_split > 1:
                    want |= {(b, h, t, c) for c in range(n_split)}
                else:
                    want.add((b, h, t, -1))
    assert set(seen) == want
    return seen, order, n_split


@pytest.mark.parametrize("B,Hq,Hkv,N,last_q,chunk", [
    (1, 32, 8, 8192, 128, 16), (1, 32, 8, 131072, 128, 64), (2, 6, 3, 1000, 300, 3),
    (1, 4, 1, 129, 1, 1), (3, 7, 7, 640, 0, 4), (1, 28, 4, 3000, 128, 8), (1, 2, 2, 64, 64, 2)])
def test_split_schedule_covers_every_chunk_once(B, Hq, Hkv, N, last_q, chunk):
    seen, order, n_split = _cover_split(B, Hq, Hkv, N, last_q, chunk)
    if n_split > 1:
        # the chunk items of the heavy tiles come first: no chunk item sits in a
        # later row of positions (blocks 8 * streams_per_xcd * group apart)
        # than a whole-row item
        groups = B * Hkv
        streams = 8 // math.gcd(groups, 8)
        per_row = 8 * (groups * streams // 8) * (Hq // Hkv)
        rows_c = [bid // per_row for bid, _, _, _, c in order if c >= 0]
        rows_n = [bid // per_row for bid, _, _, _, c in order if c < 0]
        assert not rows_n or max(rows_c) <= min(rows_n)


def test_split_workspace_size_and_arguments():
    lib = tsa.load()
    t = _good_tensors(B=1, Hq=4, Hkv=2, N=1000, d=128)
    mp = tsa.mask_params(1000, "triangle", 16, 128, 64)
    n = ctypes.c_int64()
    assert lib.tri_attn_split_workspace_size(ctypes.byref(t), ctypes.byref(mp), 4, ctypes.byref(n)) == tsa.TRI_OK
    # one heavy tile (rows 936..999 sit in tile 7), ceil(16 / 4) = 4 chunks,
    # per chunk 128 rows x (3 statistics + 128 channels) f32
    items = 1 * 4 * 1 * 4
    assert n.value == -(-items * 3 * 128 * 4 // 256) * 256 + -(-items * 128 * 128 * 4 // 256) * 256
    assert tsa.tri_attn_split_workspace_size(t, mp, 4) == n.value
    assert tsa.tri_attn_split_workspace_size(t, tsa.mask_params(1000, "triangle", 16, 128, 0), 4) == 0
    for bad in (0, -3):
        assert lib.tri_attn_split_workspace_size(ctypes.byref(t), ctypes.byref(mp), bad,
                                                 ctypes.byref(n)) == tsa.TRI_ERR_INVALID
    causal = tsa.mask_params(1000, "causal")
    assert lib.tri_attn_split_workspace_size(ctypes.byref(t), ctypes.byref(causal), 4,
                                             ctypes.byref(n)) == tsa.TRI_ERR_INVALID
    # launch-side validation, all before any HIP call
    dev = 1 << 24
    need = tsa.tri_attn_split_workspace_size(t, mp, 4)
    call = lambda mp_, hs, hw, ws, nbytes, chunk=4: lib.tri_attn_prefill_split(
        ctypes.byref(t), ctypes.byref(mp_), hs, hw, dev, dev, dev, chunk, ws, nbytes, None)
    assert call(mp, None, None, dev, need - 1) == tsa.TRI_ERR_CAPACITY
    assert call(mp, None, None, None, need) == tsa.TRI_ERR_INVALID
    assert call(mp, None, None, dev + 128, need) == tsa.TRI_ERR_INVALID          # not 256-aligned
    assert call(mp, dev, None, dev, need) == tsa.TRI_ERR_INVALID                  # sink without window
    assert call(mp, None, None, dev, need, chunk=0) == tsa.TRI_ERR_INVALID
    assert call(causal, None, None, dev, need) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_prefill_split(ctypes.byref(t), ctypes.byref(mp), None, None, None, dev, dev, 4,
                                      dev, need, None) == tsa.TRI_ERR_INVALID
    other = tsa.mask_params(999, "triangle", 16, 128, 64)
    assert call(other, None, None, dev, need) == tsa.TRI_ERR_INVALID
    z = _good_tensors(N=0)
    mz = tsa.mask_params(0, "triangle", 16, 128, 64)
    assert lib.tri_attn_prefill_split(ctypes.byref(z), ctypes.byref(mz), None, None, dev, dev, dev, 4,
                                      None, 0, None) == tsa.TRI_OK


def test_schedule_balances_unequal_heads_over_the_cu_rotation():
    # An XCD places its blocks on its 32 CUs in a fixed rotation (block u of
    # the XCD on CU slot u % 32).  With per-head windows cycling over the 4
    # heads of a group, every CU slot must still receive every head, so the
    # per-CU work stays within a few percent of the mean.
    N, Hq, Hkv = 32768, 32, 8
    mp = tsa.mask_params(N, "triangle", 0, 1, 128)
    window = [512 << (h % 4) for h in range(Hq)]
    rp, _, _ = tsa.tri_attn_plan_heads(mp, np.zeros(Hq, np.int64), np.asarray(window, np.int64))
    nq = N // 128
    lens = np.diff(rp.astype(np.int64)).reshape(Hq, nq)
    grid = tsa.tri_attn_work_item(1, Hq, Hkv, N, tsa.TRI_MASK_TRIANGLE, 128, 0)[3]
    work = np.zeros((8, 32))
    heads = [[set() for _ in range(32)] for _ in range(8)]
    for bid in range(grid):
        b, h, t, _ = tsa.tri_attn_work_item(1, Hq, Hkv, N, tsa.TRI_MASK_TRIANGLE, 128, bid)
        if t < 0 or t == nq - 1:      # the last-Q tiles are the same for every head
            continue
        x, u = bid % 8, bid // 8
        work[x, u % 32] += lens[h, t]
        heads[x][u % 32].add(h % 4)
    assert all(len(s) == 4 for row in heads for s in row)
    assert work.max() / work.mean() < 1.05


# ----------------------------------------------------------------- precision tiers

def test_quantize_k_sizes_and_arguments():
    lib = tsa.load()
    t = _good_tensors(B=2, Hq=4, Hkv=2, N=1000, d=128)
    nb, ns = ctypes.c_int64(), ctypes.c_int64()
    assert lib.tri_attn_quantize_k_sizes(ctypes.byref(t), ctypes.byref(nb), ctypes.byref(ns)) == tsa.TRI_OK
    assert nb.value == 2 * 2 * 1000 * 128 and ns.value == 2 * 2 * 16   # one scale per key tile: ceil(1000 / 64) = 16
    assert tsa.tri_attn_quantize_k_sizes(t) == (nb.value, ns.value)
    assert lib.tri_attn_quantize_k_sizes(ctypes.byref(t), None, ctypes.byref(ns)) == tsa.TRI_ERR_INVALID
    dev = 1 << 24
    assert lib.tri_attn_quantize_k(ctypes.byref(t), None, dev, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_quantize_k(ctypes.byref(t), dev + 8, dev, None) == tsa.TRI_ERR_INVALID  # 16-byte
    assert lib.tri_attn_quantize_k(ctypes.byref(t), dev, dev + 2, None) == tsa.TRI_ERR_INVALID  # 4-byte
    bad = _good_tensors(d=96)
    assert lib.tri_attn_quantize_k(ctypes.byref(bad), dev, dev, None) == tsa.TRI_ERR_UNSUPPORTED
    z = _good_tensors(N=0)
    assert lib.tri_attn_quantize_k(ctypes.byref(z), dev, dev, None) == tsa.TRI_OK
    # the fp4 copy: half the bytes, the same scales
    assert lib.tri_attn_quantize_k4_sizes(ctypes.byref(t), ctypes.byref(nb), ctypes.byref(ns)) == tsa.TRI_OK
    assert nb.value == 2 * 2 * 1000 * 64 and ns.value == 2 * 2 * 16
    assert tsa.tri_attn_quantize_k4_sizes(t) == (nb.value, ns.value)
    assert lib.tri_attn_quantize_k4(ctypes.byref(t), None, dev, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_quantize_k4(ctypes.byref(t), dev + 8, dev, None) == tsa.TRI_ERR_INVALID
    assert lib.tri_attn_quantize_k4(ctypes.byref(bad), dev, dev, None) == tsa.TRI_ERR_UNSUPPORTED
    assert lib.tri_attn_quantize_k4(ctypes.byref(z), dev, dev, None) == tsa.TRI_OK


def test_prefill_tiered_rejects_bad_arguments():
    lib = tsa.load()
    t = _good_tensors(B=1, Hq=4, Hkv=2, N=1000, d=128)
    mp = tsa.mask_params(1000, "triangle", 16, 128, 64)
    dev = 1 << 24
    # low_dist, k8, scale, fp4_dist, k4, scale4, row_ptr, k_tile, flags
    good = [dev, dev, dev, dev, dev, dev, dev, dev, dev]

    def call(mp_, args):
        return lib.tri_attn_prefill_tiered(ctypes.byref(t), ctypes.byref(mp_), *args, None)
    for i in (0, 1, 2, 6, 7, 8):
        args = list(good)
        args[i] = None
        assert call(mp, args) == tsa.TRI_ERR_INVALID, i
    for i in (3, 4, 5):   # the fp4 arrays go together
        args = list(good)
        args[i] = None
        assert call(mp, args) == tsa.TRI_ERR_INVALID, i
    for i, off in ((0, 2), (1, 8), (2, 2), (3, 2), (4, 8), (5, 2), (6, 2), (7, 2)):   # int32/f32 4, K copies 16
        args = list(good)
        args[i] = dev + off
        assert call(mp, args) == tsa.TRI_ERR_INVALID, i
    assert call(tsa.mask_params(1000, "causal"), good) == tsa.TRI_ERR_INVALID
    assert call(tsa.mask_params(999, "triangle", 16, 128, 64), good) == tsa.TRI_ERR_INVALID
    odd = tsa.mask_params(1000, "triangle", 16, 128, 64)
    odd.block_k = 32
    assert call(odd, good) == tsa.TRI_ERR_UNSUPPORTED
    z = _good_tensors(N=0)
    mz = tsa.mask_params(0, "triangle", 16, 128, 64)
    assert lib.tri_attn_prefill_tiered(ctypes.byref(z), ctypes.byref(mz), *good, None) == tsa.TRI_OK
    no4 = good[:3] + [None, None, None] + good[6:]
    assert lib.tri_attn_prefill_tiered(ctypes.byref(z), ctypes.byref(mz), *no4, None) == tsa.TRI_OK
