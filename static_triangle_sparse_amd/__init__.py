"""TriangleMix triangle-attention prefill for MI355X (gfx950).

Thin Python layer over libtriattn.so (C ABI in include/tri_attn.h).  PyTorch
supplies device memory and the stream; the tile planner and the attention
kernel run in the library.  There is no fallback path: if the library is not
built, importing the binding raises.

    from static_triangle_sparse_amd import prefill
    o, lse = prefill(q, k, v, mode="triangle", sink=128, window=2048, last_q=128)

q: [B, Hq, N, d] bf16 CUDA tensor, k/v: [B, Hkv, N, d] (any strides with the
channel axis contiguous).  Returns o [B, Hq, N, d] (bf16 or f32) and the
natural-log LSE [B, Hq, N] (f32).
"""
from __future__ import annotations

import math
import os

import numpy as np

from ._abi import (  # noqa: F401
    TRI_DTYPE_BF16, TRI_DTYPE_F32, TRI_ERR_CAPACITY, TRI_ERR_HIP, TRI_ERR_INVALID,
    TRI_ERR_UNSUPPORTED, TRI_KERNEL_BLOCK_K, TRI_KERNEL_BLOCK_Q, TRI_MASK_CAUSAL,
    TRI_MASK_TRIANGLE, TRI_OK, TRI_TILE_FULL, TRI_TILE_PARTIAL, TRI_DYN_PROBES, AttnTensors,
    DynParams, MaskParams, TriAttnError, dense_causal_prefill, last_error, load, mask_params,
    tri_attn_abi_version, tri_attn_plan, tri_attn_plan_heads, tri_attn_prefill,
    tri_attn_prefill_heads, tri_attn_prefill_lists, tri_attn_prefill_tiered,
    tri_attn_quantize_k, tri_attn_quantize_k_sizes, tri_attn_work_item, tri_dyn_plan,
    tri_dyn_plan_sizes, tri_attn_prefill_split, tri_attn_split_work_item,
    tri_attn_split_workspace_size, tri_attn_quantize_k4, tri_attn_quantize_k4_sizes,
    tri_attn_check_plan, tri_dyn_plan_noalloc, TRI_DYN_SCRATCH_BYTES,
)

__all__ = [
    "prefill", "DevicePlan", "device_plan", "make_tensors", "tri_attn_plan", "tri_attn_prefill",
    "dense_causal_prefill", "mask_params", "TriAttnError", "last_error", "layer_mode",
    "DynPlan", "dyn_plan", "tri_dyn_plan", "tri_dyn_plan_sizes", "tri_attn_prefill_lists",
    "HeadPlan", "head_plan", "tri_attn_plan_heads", "tri_attn_prefill_heads",
    "QuantizedK", "quantize_k", "tri_attn_quantize_k", "tri_attn_prefill_tiered",
    "split_workspace", "tri_attn_prefill_split", "tri_attn_split_workspace_size",
    "tri_attn_check_plan", "stack_prefill", "tri_dyn_plan_noalloc",
]

_WORKSPACE = {}


def split_workspace(nbytes: int, device, stream=None):
    """A device workspace of at least ``nbytes`` for split launches on
    ``stream`` (a torch stream; default: the device's current stream), kept
    for the life of the process and grown on demand, so that it outlives
    every launch enqueued with it.  One per (device, stream): launches on one
    stream are ordered, while launches on two streams sharing one workspace
    would overwrite each other's partials."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (str(device), int(stream.cuda_stream))
    ws = _WORKSPACE.get(key)
    if ws is None or ws.numel() < nbytes:
        # torch's caching allocator returns 512-byte-aligned blocks
        ws = torch.empty(max(256, nbytes), dtype=torch.uint8, device=device)
        _WORKSPACE[key] = ws
    return ws


def _check_plans() -> bool:
    """TRI_ATTN_CHECK_PLANS=1: every host plan built here is checked with
    tri_attn_check_plan before its device copy is made."""
    return os.environ.get("TRI_ATTN_CHECK_PLANS", "0") not in ("", "0")


def layer_mode(layer: int, tri_start: int) -> str:
    """TriangleMix layer policy: layers before ``tri_start`` stay dense causal,
    the rest use the triangle pattern (TriangleMix blog, "性能": 12 dense layers
    suffice for the Llama-3 models, 20 for Qwen2.5)."""
    return "causal" if layer < tri_start else "triangle"


class DevicePlan:
    """Host plan (numpy) plus its device copy (torch int32/uint8 tensors)."""

    def __init__(self, mp: MaskParams, device):
        import torch
        self.mp = mp
        self.row_ptr, self.k_tile, self.flags = tri_attn_plan(mp)
        if _check_plans():
            tri_attn_check_plan(mp, self.row_ptr, self.k_tile, self.flags)
        self.d_row_ptr = torch.from_numpy(self.row_ptr).to(device)
        # never hand the kernel an empty allocation
        n = max(1, self.k_tile.size)
        self.d_k_tile = torch.zeros(n, dtype=torch.int32, device=device)
        self.d_flags = torch.zeros(n, dtype=torch.uint8, device=device)
        if self.k_tile.size:
            self.d_k_tile.copy_(torch.from_numpy(self.k_tile))
            self.d_flags.copy_(torch.from_numpy(self.flags))

    @property
    def nnz(self) -> int:
        return int(self.k_tile.size)


_PLAN_CACHE = {}


def device_plan(seqlen, kind="triangle", sink=0, window=1, last_q=0, device="cuda") -> DevicePlan:
    mp = mask_params(seqlen, kind, sink, window, last_q)
    key = (mp.seqlen, mp.kind, mp.sink, mp.window, mp.last_q, str(device))
    p = _PLAN_CACHE.get(key)
    if p is None:
        p = DevicePlan(mp, device)
        _PLAN_CACHE[key] = p
    return p


def make_tensors(q, k, v, o, lse=None, scale=None) -> AttnTensors:
    """Descriptor of torch tensors q, k, v [B,H,N,d] (bf16), o (bf16/f32), lse (f32)."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
        if x.dim() != 4 or x.stride(3) != 1:
            raise ValueError(f"{name} must be 4-D [B, H, N, d] with a contiguous last axis")
    if o.dtype not in (torch.bfloat16, torch.float32) or o.stride(3) != 1:
        raise ValueError("o must be bf16 or f32 with a contiguous last axis")
    B, Hq, N, d = q.shape
    t = AttnTensors()
    t.q, t.k, t.v, t.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    t.lse = lse.data_ptr() if lse is not None else None
    t.batch, t.heads_q, t.heads_kv, t.head_dim = B, Hq, k.shape[1], d
    t.seqlen = N
    for field, x in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        getattr(t, field)[:] = [x.stride(0), x.stride(1), x.stride(2)]
    if lse is not None:
        if lse.dtype != torch.float32 or lse.stride(2) != 1:
            raise ValueError("lse must be f32 [B, Hq, N] with a contiguous last axis")
        t.lse_stride[:] = [lse.stride(0), lse.stride(1)]
    t.softmax_scale = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    t.o_dtype = TRI_DTYPE_BF16 if o.dtype == torch.bfloat16 else TRI_DTYPE_F32
    return t


class HeadPlan:
    """Per-head triangle plan (host numpy + device tensors) and the device
    per-head boundary arrays."""

    def __init__(self, seqlen, sink, window, last_q, device):
        import torch
        self.mp = mask_params(seqlen, "triangle", 0, 1, last_q)
        self.sink = np.asarray(sink, dtype=np.int64)
        self.window = np.asarray(window, dtype=np.int64)
        self.row_ptr, self.k_tile, self.flags = tri_attn_plan_heads(self.mp, self.sink, self.window)
        if _check_plans():
            tri_attn_check_plan(self.mp, self.row_ptr, self.k_tile, self.flags, self.sink, self.window)
        self.heads = int(self.sink.size)
        self.seqlen = int(seqlen)
        self.d_row_ptr = torch.from_numpy(self.row_ptr).to(device)
        n = max(1, self.k_tile.size)
        self.d_k_tile = torch.zeros(n, dtype=torch.int32, device=device)
        self.d_flags = torch.zeros(n, dtype=torch.uint8, device=device)
        if self.k_tile.size:
            self.d_k_tile.copy_(torch.from_numpy(self.k_tile))
            self.d_flags.copy_(torch.from_numpy(self.flags))
        clip = lambda x: np.minimum(x, np.iinfo(np.int32).max).astype(np.int32)
        self.d_sink = torch.from_numpy(clip(self.sink)).to(device)
        self.d_window = torch.from_numpy(clip(self.window)).to(device)


def head_plan(seqlen, sink, window, last_q=0, device="cuda") -> HeadPlan:
    """Triangle plan with per-head sink and window (one value per query head)."""
    return HeadPlan(seqlen, sink, window, last_q, device)


class QuantizedK:
    """fp8 copy of K for the precision tiers (device uint8 k8, f32 scales),
    and with fp4=True also the fp4 copy (k4, scale4)."""

    def __init__(self, t: AttnTensors, device, fp4: bool = False):
        import torch
        # the K it was made for: (batch, heads_kv, seqlen, head_dim)
        self.shape = (int(t.batch), int(t.heads_kv), int(t.seqlen), int(t.head_dim))
        nbytes, nscales = tri_attn_quantize_k_sizes(t)
        self.k8 = torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)
        self.scale = torch.empty(max(1, nscales), dtype=torch.float32, device=device)
        self.k4 = self.scale4 = None
        if fp4:
            nbytes4, nscales4 = tri_attn_quantize_k4_sizes(t)
            self.k4 = torch.empty(max(16, nbytes4), dtype=torch.uint8, device=device)
            self.scale4 = torch.empty(max(1, nscales4), dtype=torch.float32, device=device)

    def run(self, t: AttnTensors, stream: int) -> None:
        if (t.batch, t.heads_kv, t.seqlen, t.head_dim) != self.shape:
            raise ValueError(f"QuantizedK sized for K {self.shape}, called on "
                             f"{(t.batch, t.heads_kv, t.seqlen, t.head_dim)}")
        tri_attn_quantize_k(t, self.k8.data_ptr(), self.scale.data_ptr(), stream)
        if self.k4 is not None:
            tri_attn_quantize_k4(t, self.k4.data_ptr(), self.scale4.data_ptr(), stream)


def quantize_k(q, k, stream=None, fp4=False) -> QuantizedK:
    """fp8 (e4m3) copy of k in the tiered kernel's layout, with its scales
    (and the fp4 (e2m1) copy with fp4=True)."""
    import torch
    o = torch.empty((1, 1, 1, 8), dtype=torch.bfloat16, device=k.device)  # not written
    t = make_tensors(q, k, k, o, None)
    qk = QuantizedK(t, k.device, fp4)
    s = (stream if stream is not None else torch.cuda.current_stream(k.device)).cuda_stream
    qk.run(t, s)
    return qk


class DynPlan:
    """Device buffers of a dynamic block-sparse plan (tri_dyn_plan): workspace,
    row_ptr [n_rows + 1], k_tile and flags [max_nnz], all torch tensors."""

    def __init__(self, t: AttnTensors, device):
        import torch
        self.workspace_bytes, self.n_rows, self.max_nnz = tri_dyn_plan_sizes(t)
        # the layer it lists: (batch, heads_q, seqlen)
        self.shape = (int(t.batch), int(t.heads_q), int(t.seqlen))
        # torch's caching allocator returns 512-byte-aligned blocks
        self.workspace = torch.empty(max(256, self.workspace_bytes), dtype=torch.uint8, device=device)
        self.d_row_ptr = torch.empty(self.n_rows + 1, dtype=torch.int32, device=device)
        self.d_k_tile = torch.empty(max(1, self.max_nnz), dtype=torch.int32, device=device)
        self.d_flags = torch.empty(max(1, self.max_nnz), dtype=torch.uint8, device=device)

    def run(self, t: AttnTensors, alpha: float, stream: int) -> None:
        if (t.batch, t.heads_q, t.seqlen) != self.shape:
            raise ValueError(f"DynPlan sized for (B, Hq, N) = {self.shape}, called on "
                             f"{(t.batch, t.heads_q, t.seqlen)}")
        tri_dyn_plan(t, alpha, self.workspace.data_ptr(), self.workspace.numel(),
                     self.d_row_ptr.data_ptr(), self.d_k_tile.data_ptr(), self.d_flags.data_ptr(),
                     self.d_k_tile.numel(), stream)


def dyn_plan(q, k, alpha, scale=None, stream=None) -> DynPlan:
    """Dynamic tile lists of a dense layer (FlashPrefill-style probe selection)."""
    import torch
    # the selection reads q and k only; o is a placeholder the call never writes
    o = torch.empty((1, 1, 1, 8), dtype=torch.bfloat16, device=q.device)
    t = make_tensors(q, k, k, o, None, scale)
    p = DynPlan(t, q.device)
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    p.run(t, alpha, s)
    return p


def _per_head(x, Hq: int, name: str) -> np.ndarray:
    """One int32 value per query head (clipped to the int32 range); anything
    else is rejected, since the kernel reads entry h for every query head h."""
    a = np.asarray(x, np.int64)
    if a.ndim != 1 or a.size != Hq:
        raise ValueError(f"{name} must hold one value per query head ({Hq}), got shape {a.shape}")
    return np.clip(a, np.iinfo(np.int32).min, np.iinfo(np.int32).max).astype(np.int32)


def _check_head_plan(plan, Hq: int, N: int) -> None:
    if not isinstance(plan, HeadPlan):
        raise ValueError("mode 'triangle_heads' needs plan= (a HeadPlan)")
    if plan.heads != Hq or plan.seqlen != N:
        raise ValueError(f"HeadPlan made for {plan.heads} heads and N = {plan.seqlen}, "
                         f"the layer has {Hq} heads and N = {N}")


def prefill(q, k, v, mode="triangle", sink=0, window=1, last_q=0, o_dtype=None, scale=None,
            out=None, lse=None, stream=None, plan=None, low_dist=None, split=None, fp4_dist=None):
    """One attention layer on the GPU; returns (o, lse).  ``mode`` is
    "triangle" (planned tile list), "triangle_heads" (a HeadPlan), "tiered"
    (fp8 far tiles; ``low_dist`` and ``fp4_dist`` hold one boundary per query
    head), "causal" (dense layer) or "lists" (per-head tile lists of a
    DynPlan, causal mask inside the tiles).  ``split``: for "triangle" and
    "triangle_heads", walk the last-Q rows in chunks of this many key tiles on
    separate workgroups (tri_attn_prefill_split)."""
    import torch
    B, Hq, N, d = q.shape
    if o_dtype is None:
        o_dtype = torch.bfloat16
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    t = make_tensors(q, k, v, out, lse, scale)
    torch_stream = stream if stream is not None else torch.cuda.current_stream(q.device)
    s = torch_stream.cuda_stream
    if split is not None and mode not in ("triangle", "triangle_heads"):
        raise ValueError("split= applies to modes 'triangle' and 'triangle_heads'")
    if split is not None:
        if mode == "triangle":
            p = device_plan(N, "triangle", sink, window, last_q, q.device)
            heads = (None, None)
        else:
            _check_head_plan(plan, Hq, N)
            p = plan
            heads = (plan.d_sink.data_ptr(), plan.d_window.data_ptr())
        nbytes = tri_attn_split_workspace_size(t, p.mp, int(split))
        ws = split_workspace(nbytes, q.device, torch_stream)
        tri_attn_prefill_split(t, p.mp, heads[0], heads[1], p.d_row_ptr.data_ptr(),
                               p.d_k_tile.data_ptr(), p.d_flags.data_ptr(), int(split), ws.data_ptr(),
                               ws.numel(), s)
    elif mode == "causal":
        dense_causal_prefill(t, s)
    elif mode == "triangle":
        p = device_plan(N, "triangle", sink, window, last_q, q.device)
        tri_attn_prefill(t, p.mp, p.d_row_ptr.data_ptr(), p.d_k_tile.data_ptr(),
                         p.d_flags.data_ptr(), s)
    elif mode == "triangle_heads":
        _check_head_plan(plan, Hq, N)
        tri_attn_prefill_heads(t, plan.mp, plan.d_sink.data_ptr(), plan.d_window.data_ptr(),
                               plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                               plan.d_flags.data_ptr(), s)
    elif mode == "tiered":
        if not isinstance(plan, QuantizedK) or low_dist is None:
            raise ValueError("mode 'tiered' needs plan= (a QuantizedK of k) and low_dist=")
        kshape = (B, k.shape[1], N, d)
        if plan.shape != kshape:
            raise ValueError(f"QuantizedK made for K {plan.shape}, this layer's K is {kshape}")
        p = device_plan(N, "triangle", sink, window, last_q, q.device)
        # the device copy of the boundaries lives on the QuantizedK object, so it
        # outlives the enqueued kernel
        plan.low_dist = torch.from_numpy(_per_head(low_dist, Hq, "low_dist")).to(q.device)
        fp4_args = (None, None, None)
        if fp4_dist is not None:
            if plan.k4 is None:
                raise ValueError("fp4_dist= needs a QuantizedK made with fp4=True")
            plan.fp4_dist = torch.from_numpy(_per_head(fp4_dist, Hq, "fp4_dist")).to(q.device)
            fp4_args = (plan.fp4_dist.data_ptr(), plan.k4.data_ptr(), plan.scale4.data_ptr())
        tri_attn_prefill_tiered(t, p.mp, plan.low_dist.data_ptr(), plan.k8.data_ptr(),
                                plan.scale.data_ptr(), *fp4_args, p.d_row_ptr.data_ptr(),
                                p.d_k_tile.data_ptr(), p.d_flags.data_ptr(), s)
    elif mode == "lists":
        if not isinstance(plan, DynPlan):
            raise ValueError("mode 'lists' needs plan= (a DynPlan)")
        if plan.shape != (B, Hq, N):
            raise ValueError(f"DynPlan made for (B, Hq, N) = {plan.shape}, the layer is {(B, Hq, N)}")
        tri_attn_prefill_lists(t, plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                               plan.d_flags.data_ptr(), s)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return out, lse


def stack_prefill(layers, tri_start, sink, window, last_q, stream=None):
    """Attention of a TriangleMix layer stack, enqueued layer after layer on
    one stream: layer l runs dense causal if l < tri_start, else the triangle
    pattern with (sink, window, last_q) (``layer_mode``).  ``layers`` is a
    sequence of AttnTensors descriptors (make_tensors) of equal seqlen;
    returns the mode each layer ran in."""
    import torch
    if not layers:
        return []
    N = int(layers[0].seqlen)
    if any(int(t.seqlen) != N for t in layers):
        raise ValueError("every layer of a stack has the same sequence length")
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    p = None
    modes = [layer_mode(l, tri_start) for l in range(len(layers))]
    for t, m in zip(layers, modes):
        if m == "causal":
            dense_causal_prefill(t, s)
        else:
            if p is None:
                p = device_plan(N, "triangle", sink, window, last_q, torch.cuda.current_device())
            tri_attn_prefill(t, p.mp, p.d_row_ptr.data_ptr(), p.d_k_tile.data_ptr(),
                             p.d_flags.data_ptr(), s)
    return modes
