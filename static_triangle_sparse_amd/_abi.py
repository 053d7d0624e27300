"""ctypes binding of libtriattn.so (include/tri_attn.h).

Argument marshalling only: every step of the attention path runs in the
library (host planner, gfx950 kernel).  The structures below mirror the C
header field by field.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# TRI_ATTN_LIB names another build of the same library; only the host-only
# sanitizer build of the test suite sets it
LIB_PATH = os.environ.get("TRI_ATTN_LIB") or os.path.join(_PKG, "libtriattn.so")

TRI_OK = 0
TRI_ERR_INVALID = -1
TRI_ERR_CAPACITY = -2
TRI_ERR_UNSUPPORTED = -3
TRI_ERR_HIP = -4

TRI_MASK_TRIANGLE = 0
TRI_MASK_CAUSAL = 1
TRI_DTYPE_BF16 = 0
TRI_DTYPE_F32 = 1
TRI_TILE_FULL = 0
TRI_TILE_PARTIAL = 1
TRI_KERNEL_BLOCK_Q = 128
TRI_KERNEL_BLOCK_K = 64
TRI_DYN_PROBES = 16
TRI_DYN_SCRATCH_BYTES = 64 << 20

_STATUS_NAMES = {
    TRI_OK: "TRI_OK", TRI_ERR_INVALID: "TRI_ERR_INVALID", TRI_ERR_CAPACITY: "TRI_ERR_CAPACITY",
    TRI_ERR_UNSUPPORTED: "TRI_ERR_UNSUPPORTED", TRI_ERR_HIP: "TRI_ERR_HIP",
}


class TriAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class MaskParams(ctypes.Structure):
    _fields_ = [
        ("seqlen", ctypes.c_int64),
        ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("sink", ctypes.c_int64),
        ("window", ctypes.c_int64),
        ("last_q", ctypes.c_int64),
    ]


class AttnTensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seqlen", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("lse_stride", ctypes.c_int64 * 2),
        ("softmax_scale", ctypes.c_float),
        ("o_dtype", ctypes.c_int32),
    ]


class DynParams(ctypes.Structure):
    _fields_ = [
        ("alpha", ctypes.c_float),
        ("n_probe", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m static_triangle_sparse_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.tri_attn_plan.argtypes = [P(MaskParams), P(ctypes.c_int32), P(ctypes.c_int32),
                                  P(ctypes.c_uint8), ctypes.c_int64, P(ctypes.c_int32),
                                  P(ctypes.c_int64)]
    lib.tri_attn_plan.restype = ctypes.c_int
    lib.tri_attn_check_plan.argtypes = [P(MaskParams), ctypes.c_int32, P(ctypes.c_int64),
                                        P(ctypes.c_int64), P(ctypes.c_int32), ctypes.c_int64,
                                        P(ctypes.c_int32), P(ctypes.c_uint8), ctypes.c_int64]
    lib.tri_attn_check_plan.restype = ctypes.c_int
    lib.tri_attn_prefill.argtypes = [P(AttnTensors), P(MaskParams), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.tri_attn_prefill.restype = ctypes.c_int
    lib.dense_causal_prefill.argtypes = [P(AttnTensors), ctypes.c_void_p]
    lib.dense_causal_prefill.restype = ctypes.c_int
    lib.tri_attn_last_error.argtypes = []
    lib.tri_attn_last_error.restype = ctypes.c_char_p
    lib.tri_attn_abi_version.argtypes = []
    lib.tri_attn_abi_version.restype = ctypes.c_int
    lib.tri_attn_work_item.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int64, P(ctypes.c_int32), P(ctypes.c_int32),
                                       P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.tri_attn_work_item.restype = ctypes.c_int
    lib.tri_dyn_plan_sizes.argtypes = [P(AttnTensors), P(ctypes.c_int64), P(ctypes.c_int64),
                                       P(ctypes.c_int64)]
    lib.tri_dyn_plan_sizes.restype = ctypes.c_int
    lib.tri_dyn_plan.argtypes = [P(AttnTensors), P(DynParams), ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p]
    lib.tri_dyn_plan.restype = ctypes.c_int
    lib.tri_dyn_plan_noalloc.argtypes = [P(AttnTensors), P(DynParams), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.tri_dyn_plan_noalloc.restype = ctypes.c_int
    lib.tri_attn_prefill_lists.argtypes = [P(AttnTensors), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    lib.tri_attn_prefill_lists.restype = ctypes.c_int
    lib.tri_attn_plan_heads.argtypes = [P(MaskParams), ctypes.c_int32, P(ctypes.c_int64),
                                        P(ctypes.c_int64), P(ctypes.c_int32), P(ctypes.c_int32),
                                        P(ctypes.c_uint8), ctypes.c_int64, P(ctypes.c_int32),
                                        P(ctypes.c_int64)]
    lib.tri_attn_plan_heads.restype = ctypes.c_int
    lib.tri_attn_prefill_heads.argtypes = [P(AttnTensors), P(MaskParams), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    lib.tri_attn_prefill_heads.restype = ctypes.c_int
    lib.tri_attn_quantize_k_sizes.argtypes = [P(AttnTensors), P(ctypes.c_int64), P(ctypes.c_int64)]
    lib.tri_attn_quantize_k_sizes.restype = ctypes.c_int
    lib.tri_attn_quantize_k.argtypes = [P(AttnTensors), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.tri_attn_quantize_k.restype = ctypes.c_int
    lib.tri_attn_prefill_tiered.argtypes = [P(AttnTensors), P(MaskParams), ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.tri_attn_quantize_k4_sizes.argtypes = [P(AttnTensors), P(ctypes.c_int64), P(ctypes.c_int64)]
    lib.tri_attn_quantize_k4_sizes.restype = ctypes.c_int
    lib.tri_attn_quantize_k4.argtypes = [P(AttnTensors), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.tri_attn_quantize_k4.restype = ctypes.c_int
    lib.tri_attn_prefill_tiered.restype = ctypes.c_int
    lib.tri_attn_split_workspace_size.argtypes = [P(AttnTensors), P(MaskParams), ctypes.c_int32,
                                                  P(ctypes.c_int64)]
    lib.tri_attn_split_workspace_size.restype = ctypes.c_int
    lib.tri_attn_prefill_split.argtypes = [P(AttnTensors), P(MaskParams), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_void_p]
    lib.tri_attn_prefill_split.restype = ctypes.c_int
    lib.tri_attn_split_work_item.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int64, P(ctypes.c_int32), P(ctypes.c_int32),
                                             P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.tri_attn_split_work_item.restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().tri_attn_last_error().decode()


def _check(status: int) -> None:
    if status != TRI_OK:
        raise TriAttnError(status, last_error())


def mask_params(seqlen, kind=TRI_MASK_TRIANGLE, sink=0, window=1, last_q=0,
                block_q=TRI_KERNEL_BLOCK_Q, block_k=TRI_KERNEL_BLOCK_K) -> MaskParams:
    if isinstance(kind, str):
        kind = {"triangle": TRI_MASK_TRIANGLE, "causal": TRI_MASK_CAUSAL}[kind]
    return MaskParams(int(seqlen), int(block_q), int(block_k), int(kind), 0, int(sink),
                      int(window), int(last_q))


def tri_attn_plan(mp: MaskParams):
    """Host tile planner.  Returns (row_ptr int32[nq+1], k_tile int32[nnz],
    flags uint8[nnz]) as numpy arrays."""
    lib = load()
    nq = ctypes.c_int32()
    nnz = ctypes.c_int64()
    _check(lib.tri_attn_plan(ctypes.byref(mp), None, None, None, 0, ctypes.byref(nq),
                             ctypes.byref(nnz)))
    row_ptr = np.zeros(nq.value + 1, dtype=np.int32)
    k_tile = np.zeros(max(1, nnz.value), dtype=np.int32)
    flags = np.zeros(max(1, nnz.value), dtype=np.uint8)
    _check(lib.tri_attn_plan(
        ctypes.byref(mp), row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        k_tile.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        flags.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), nnz.value, ctypes.byref(nq),
        ctypes.byref(nnz)))
    return row_ptr, k_tile[:nnz.value], flags[:nnz.value]


def tri_attn_check_plan(mp: MaskParams, row_ptr, k_tile, flags, sink=None, window=None) -> None:
    """Host check of a plan (tri_attn_check_plan); raises TriAttnError when
    the arrays are not a valid plan for ``mp`` (per-head ``sink``/``window``:
    the layout of tri_attn_plan_heads)."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    k_tile = np.ascontiguousarray(k_tile, dtype=np.int32)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    if k_tile.size != flags.size:
        raise ValueError("k_tile and flags must have the same length")
    heads, ps, pw = 0, None, None
    P64 = ctypes.POINTER(ctypes.c_int64)
    if sink is not None or window is not None:
        sink = np.ascontiguousarray(sink, dtype=np.int64)
        window = np.ascontiguousarray(window, dtype=np.int64)
        if sink.shape != window.shape or sink.ndim != 1:
            raise ValueError("sink and window must be 1-D of the same length")
        heads, ps, pw = sink.size, sink.ctypes.data_as(P64), window.ctypes.data_as(P64)
    _check(load().tri_attn_check_plan(
        ctypes.byref(mp), heads, ps, pw, row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        row_ptr.size - 1, k_tile.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        flags.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), k_tile.size))


def tri_attn_prefill(t: AttnTensors, mp: MaskParams, d_row_ptr: int, d_k_tile: int,
                     d_flags: int, stream: int) -> None:
    """Enqueue a planned (triangle) layer; pointers are device addresses."""
    _check(load().tri_attn_prefill(ctypes.byref(t), ctypes.byref(mp), d_row_ptr, d_k_tile,
                                   d_flags, stream))


def dense_causal_prefill(t: AttnTensors, stream: int) -> None:
    """Enqueue a dense causal layer."""
    _check(load().dense_causal_prefill(ctypes.byref(t), stream))


def tri_attn_abi_version() -> int:
    return load().tri_attn_abi_version()


def tri_attn_work_item(batch, heads_q, heads_kv, seqlen, kind, last_q, bid):
    """(b, h, qtile, grid) of launch block ``bid`` (qtile -1: idle block)."""
    b = ctypes.c_int32()
    h = ctypes.c_int32()
    t = ctypes.c_int32()
    grid = ctypes.c_int64()
    _check(load().tri_attn_work_item(batch, heads_q, heads_kv, seqlen, kind, last_q, bid,
                                     ctypes.byref(b), ctypes.byref(h), ctypes.byref(t),
                                     ctypes.byref(grid)))
    return b.value, h.value, t.value, grid.value


def tri_dyn_plan_sizes(t: AttnTensors):
    """(workspace_bytes, n_rows, max_nnz) of the dynamic plan of layer ``t``."""
    ws = ctypes.c_int64()
    rows = ctypes.c_int64()
    nnz = ctypes.c_int64()
    _check(load().tri_dyn_plan_sizes(ctypes.byref(t), ctypes.byref(ws), ctypes.byref(rows),
                                     ctypes.byref(nnz)))
    return ws.value, rows.value, nnz.value


def tri_dyn_plan(t: AttnTensors, alpha: float, d_workspace: int, workspace_bytes: int,
                 d_row_ptr: int, d_k_tile: int, d_flags: int, capacity: int, stream: int,
                 n_probe: int = TRI_DYN_PROBES) -> None:
    """Enqueue the dynamic tile selection; pointers are device addresses."""
    dp = DynParams(float(alpha), int(n_probe))
    _check(load().tri_dyn_plan(ctypes.byref(t), ctypes.byref(dp), d_workspace, workspace_bytes,
                               d_row_ptr, d_k_tile, d_flags, capacity, stream))


def tri_dyn_plan_noalloc(t: AttnTensors, alpha: float, d_row_ptr: int, d_k_tile: int, d_flags: int,
                         capacity: int, stream: int, n_probe: int = TRI_DYN_PROBES) -> None:
    """tri_dyn_plan with the library-owned workspace (no allocation); device
    output pointers as for tri_dyn_plan."""
    dp = DynParams(float(alpha), int(n_probe))
    _check(load().tri_dyn_plan_noalloc(ctypes.byref(t), ctypes.byref(dp), d_row_ptr, d_k_tile, d_flags,
                                       capacity, stream))


def tri_attn_prefill_lists(t: AttnTensors, d_row_ptr: int, d_k_tile: int, d_flags: int,
                           stream: int) -> None:
    """Enqueue attention over per-(batch, head) tile lists."""
    _check(load().tri_attn_prefill_lists(ctypes.byref(t), d_row_ptr, d_k_tile, d_flags, stream))


def tri_attn_plan_heads(mp: MaskParams, sink, window):
    """Host planner with per-head (sink, window).  Returns (row_ptr
    int32[H*nq+1], k_tile int32[nnz], flags uint8[nnz]) over rows h*nq + t."""
    lib = load()
    sink = np.ascontiguousarray(sink, dtype=np.int64)
    window = np.ascontiguousarray(window, dtype=np.int64)
    if sink.shape != window.shape or sink.ndim != 1:
        raise ValueError("sink and window must be 1-D of the same length")
    H = sink.size
    P64 = ctypes.POINTER(ctypes.c_int64)
    nq = ctypes.c_int32()
    nnz = ctypes.c_int64()
    _check(lib.tri_attn_plan_heads(ctypes.byref(mp), H, sink.ctypes.data_as(P64),
                                   window.ctypes.data_as(P64), None, None, None, 0,
                                   ctypes.byref(nq), ctypes.byref(nnz)))
    row_ptr = np.zeros(H * nq.value + 1, dtype=np.int32)
    k_tile = np.zeros(max(1, nnz.value), dtype=np.int32)
    flags = np.zeros(max(1, nnz.value), dtype=np.uint8)
    _check(lib.tri_attn_plan_heads(
        ctypes.byref(mp), H, sink.ctypes.data_as(P64), window.ctypes.data_as(P64),
        row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        k_tile.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        flags.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), nnz.value, ctypes.byref(nq),
        ctypes.byref(nnz)))
    return row_ptr, k_tile[:nnz.value], flags[:nnz.value]


def tri_attn_prefill_heads(t: AttnTensors, mp: MaskParams, d_head_sink: int, d_head_window: int,
                           d_row_ptr: int, d_k_tile: int, d_flags: int, stream: int) -> None:
    """Enqueue a triangle layer with per-head boundaries (device pointers)."""
    _check(load().tri_attn_prefill_heads(ctypes.byref(t), ctypes.byref(mp), d_head_sink,
                                         d_head_window, d_row_ptr, d_k_tile, d_flags, stream))


def tri_attn_quantize_k_sizes(t: AttnTensors):
    """(bytes of the fp8 K, number of f32 scales) for layer ``t``."""
    nb = ctypes.c_int64()
    ns = ctypes.c_int64()
    _check(load().tri_attn_quantize_k_sizes(ctypes.byref(t), ctypes.byref(nb), ctypes.byref(ns)))
    return nb.value, ns.value


def tri_attn_quantize_k(t: AttnTensors, d_k8: int, d_scale: int, stream: int) -> None:
    """Enqueue the fp8 copy of t.k (device pointers)."""
    _check(load().tri_attn_quantize_k(ctypes.byref(t), d_k8, d_scale, stream))


def tri_attn_prefill_tiered(t: AttnTensors, mp: MaskParams, d_low_dist: int, d_k8: int,
                            d_scale: int, d_fp4_dist, d_k4, d_scale4, d_row_ptr: int, d_k_tile: int,
                            d_flags: int, stream: int) -> None:
    """Enqueue a triangle layer with fp8 (and fp4: the three fp4 pointers, or
    None for none) scores on far tiles (device pointers)."""
    _check(load().tri_attn_prefill_tiered(ctypes.byref(t), ctypes.byref(mp), d_low_dist, d_k8,
                                          d_scale, d_fp4_dist, d_k4, d_scale4, d_row_ptr, d_k_tile,
                                          d_flags, stream))


def tri_attn_quantize_k4_sizes(t: AttnTensors):
    """(bytes of the fp4 K, number of f32 scales) for layer ``t``."""
    nb = ctypes.c_int64()
    ns = ctypes.c_int64()
    _check(load().tri_attn_quantize_k4_sizes(ctypes.byref(t), ctypes.byref(nb), ctypes.byref(ns)))
    return nb.value, ns.value


def tri_attn_quantize_k4(t: AttnTensors, d_k4: int, d_scale: int, stream: int) -> None:
    """Enqueue the fp4 copy of t.k (device pointers)."""
    _check(load().tri_attn_quantize_k4(ctypes.byref(t), d_k4, d_scale, stream))


def tri_attn_split_workspace_size(t: AttnTensors, mp: MaskParams, chunk_tiles: int) -> int:
    """Device bytes of the workspace of a split launch (0: nothing to split)."""
    n = ctypes.c_int64()
    _check(load().tri_attn_split_workspace_size(ctypes.byref(t), ctypes.byref(mp), chunk_tiles,
                                                ctypes.byref(n)))
    return n.value


def tri_attn_prefill_split(t: AttnTensors, mp: MaskParams, d_head_sink, d_head_window, d_row_ptr: int,
                           d_k_tile: int, d_flags: int, chunk_tiles: int, d_workspace, workspace_bytes: int,
                           stream: int) -> None:
    """Enqueue a triangle layer whose last-Q rows are walked in chunks (device
    pointers; head arrays None for one shared plan)."""
    _check(load().tri_attn_prefill_split(ctypes.byref(t), ctypes.byref(mp), d_head_sink, d_head_window,
                                         d_row_ptr, d_k_tile, d_flags, chunk_tiles, d_workspace,
                                         workspace_bytes, stream))


def tri_attn_split_work_item(batch, heads_q, heads_kv, seqlen, last_q, chunk_tiles, bid):
    """(b, h, qtile, chunk, grid) of block ``bid`` of a split launch."""
    b, h, t, c = (ctypes.c_int32() for _ in range(4))
    grid = ctypes.c_int64()
    _check(load().tri_attn_split_work_item(batch, heads_q, heads_kv, seqlen, last_q, chunk_tiles, bid,
                                           ctypes.byref(b), ctypes.byref(h), ctypes.byref(t),
                                           ctypes.byref(c), ctypes.byref(grid)))
    return b.value, h.value, t.value, c.value, grid.value
