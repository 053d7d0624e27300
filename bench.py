"""Benchmark of the TriangleMix triangle-attention prefill on one MI355X.

Default workload: one Llama-3-8B-shaped attention layer (32 query heads, 8 KV
heads, head_dim 128, batch 1) at N = 131072 tokens with the triangle mask
(sink 128, window 2048, last-Q 128), bf16 Q/K/V ~ N(0, 1) from a seeded host
generator, bf16 O plus f32 LSE.  One step = one triangle layer (the planned
tile list is built once, outside the timed region).  The dense causal layer
runs on the same inputs for the triangle-vs-dense ratio.

Prints one JSON line.  ``value`` is kept-tile TFLOP/s: 4 * 128 * 64 * d FLOPs
per kept (query tile, key tile) pair per query head (partial tiles count in
full), divided by the measured time per layer.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--config 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "triangle prefill ms + kept-tile TFLOP/s (% bf16 MFMA peak) at 128K, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
KERNEL_SRC = os.path.join(ROOT, "static_triangle_sparse_amd", "csrc", "attn_fwd_gfx950.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_triangle_llama128k_traffic.txt")
TRAFFIC_CONFIG = 3  # the workload the counters in TRAFFIC_FILE were taken on

CONFIGS = {
    1: dict(name="single head, N=512, d=64 (sink 64, window 128, last-Q 64)",
            B=1, Hq=1, Hkv=1, N=512, d=64, sink=64, window=128, last_q=64, layers=None),
    2: dict(name="Llama-3-8B-shaped layer (32q/8kv, d=128), N=32768",
            B=1, Hq=32, Hkv=8, N=32768, d=128, sink=128, window=2048, last_q=128, layers=None),
    3: dict(name="Llama-3-8B-shaped layer (32q/8kv, d=128), N=131072",
            B=1, Hq=32, Hkv=8, N=131072, d=128, sink=128, window=2048, last_q=128, layers=None),
    4: dict(name="Llama-3-8B-shaped 32-layer stack, N=65536, layers 0-11 dense, 12-31 triangle",
            B=1, Hq=32, Hkv=8, N=65536, d=128, sink=128, window=2048, last_q=128,
            layers=32, tri_start=12),
    5: dict(name="Qwen2.5-7B-shaped 28-layer stack (28q/4kv), N=131072, layers 0-19 dense, 20-27 triangle",
            B=1, Hq=28, Hkv=4, N=131072, d=128, sink=128, window=2048, last_q=128,
            layers=28, tri_start=20),
}


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(config: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and on this workload; else None."""
    if config != TRAFFIC_CONFIG or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kept_tiles_per_head(plan) -> int:
    return int(plan.k_tile.size)


def causal_tiles_per_head(N: int) -> int:
    nq = -(-N // 128)
    return sum(min(N - 1, t * 128 + 127) // 64 + 1 for t in range(nq))


def make_layer_inputs(cfg, seed, dev, host=True):
    """bf16 Q, K, V on the device.  host=True: the shared seeded numpy
    generator (bit-identical to what the parity tests use); host=False: torch's
    device generator (stack benchmarks, where per-layer host generation of
    tens of GB would dominate the run)."""
    import torch
    B, Hq, Hkv, N, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["d"]
    if host:
        import synth
        bits = synth.qkv_bf16_bits(seed, B, Hq, Hkv, N, d)
        out = [torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) for x in bits]
        return out, bits
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    mk = lambda h: torch.randn((B, h, N, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return [mk(Hq), mk(Hkv), mk(Hkv)], None


def time_launches(fn, steps, warmup):
    """Average ms per launch of fn() over `steps` back-to-back launches,
    bracketed by device synchronisation; HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return start.elapsed_time(stop) / steps, wall


def time_each(fn, runs, flush_mib=0):
    """Per-launch ms of `runs` launches of fn(), each bracketed by its own HIP
    events on the launch stream.  With flush_mib, a write of that many MiB of
    scratch precedes every launch (outside the events), so each launch starts
    with K/V/Q evicted from the 256 MB Infinity Cache and the L2s."""
    import torch
    scratch = torch.empty(max(1, flush_mib) << 20, dtype=torch.uint8, device="cuda") if flush_mib else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for i, (a, b) in enumerate(ev):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    del scratch
    return {"median_ms": round(ms[len(ms) // 2], 4), "min_ms": round(ms[0], 4), "runs": runs}


def measure_clock(fn, launch_ms, seconds=2.5, skip_s=1.0):
    """Mean shader clock (MHz) of GPU 0 while fn() runs back to back for about
    `seconds`: the launches are queued, then amdsmi's per-XCD graphics clocks
    are read every 0.25 s once `skip_s` of ramp-up has passed (amdsmi refreshes
    its metrics about once a second).  Returns (mhz or None, detail)."""
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return None, f"{len(handles)} GPUs visible to amdsmi"
        h = handles[0]

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            xcd = [float(x) for x in m.get("current_gfxclks", []) if isinstance(x, (int, float))]
            if xcd:
                return sum(xcd) / len(xcd)
            return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"])
        read()
    except Exception as e:  # noqa: BLE001 - report, never fail the bench over it
        return None, f"amdsmi: {type(e).__name__}: {e}"
    n = max(1, int(seconds * 1e3 / max(launch_ms, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    samples = []
    while time.perf_counter() - t0 < seconds:
        time.sleep(0.25)
        if time.perf_counter() - t0 >= skip_s:
            samples.append(read())
    torch.cuda.synchronize()
    if not samples:
        return None, "no samples"
    return sum(samples) / len(samples), f"{len(samples)} samples over {n} launches (mean of the XCD clocks)"


def sample_tiles(N, n_random_tiles=128):
    """Query tiles of the oracle sample: {0, 1, 15, 16, 17, nq-2, nq-1} plus
    `n_random_tiles` seeded random middle tiles (15..17 straddle the 2048-key
    window edge)."""
    nq = -(-N // 128)
    rng = np.random.default_rng(1)
    middle = np.arange(18, max(18, nq - 2))
    tiles = sorted({0, 1, 15, 16, 17, nq - 2, nq - 1} |
                   set(int(x) for x in rng.choice(middle, min(n_random_tiles, middle.size),
                                                   replace=False)))
    tiles = [t for t in tiles if 0 <= t < nq]
    rows = np.concatenate([np.arange(t * 128, min(N, (t + 1) * 128)) for t in tiles])
    return tiles, rows


def cpu_baseline(bits, cfg, plan):
    """The fp64 oracle, as it stands, on a bounded sample of the same layer:
    the rows of ``sample_tiles``, all heads (10-30 s of host work at 128K).
    Returns (the cpu_baseline object, (rows, oracle O, oracle LSE))."""
    from oracle import attention as oatt
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    N, Hq, d = cfg["N"], cfg["Hq"], cfg["d"]
    tiles, rows = sample_tiles(N)
    kept = sum(int(plan.row_ptr[t + 1] - plan.row_ptr[t]) for t in tiles)
    flops = 4.0 * 128 * 64 * d * kept * Hq * cfg["B"]
    f64 = synth.bf16_bits_to_f64
    q, k, v = f64(bits[0]), f64(bits[1]), f64(bits[2])
    t0 = time.perf_counter()
    ro, rl = oatt.attention(q, k, v, "triangle", cfg["sink"], cfg["window"], cfg["last_q"], rows=rows)
    dt = time.perf_counter() - t0
    total_flops = 4.0 * 128 * 64 * d * plan.k_tile.size * Hq * cfg["B"]
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle (OpenBLAS, {threads} threads, {cpu_model or 'cpu'}) on "
                   f"{len(tiles)} query tiles (0, 1, 15-17, last two, {len(tiles) - 7} seeded random) of "
                   f"all {Hq} heads ({rows.size} rows, {kept} kept tiles/head): "
                   f"{dt:.2f} s; kept-tile FLOPs of the sample / time; full layer extrapolated "
                   f"{dt * total_flops / flops:.1f} s"),
    }, (rows, ro, rl)


def sample_of(o, lse, rows):
    """Host copy of the sample rows of a layer's outputs (O as float64)."""
    import torch
    idx = torch.from_numpy(rows).to(o.device)
    return (o[:, :, idx].float().cpu().numpy().astype(np.float64),
            lse[:, :, idx].cpu().numpy().astype(np.float64))


def full_oracle(bits, cfg, plan, tri, o, lse):
    """The fp64 oracle on every row of the layer, timed on the host, and the
    whole GPU layer (one more launch) against it."""
    import torch
    from oracle import attention as oatt
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    print("[bench] full-layer oracle ...", file=sys.stderr, flush=True)
    f64 = synth.bf16_bits_to_f64
    q, k, v = f64(bits[0]), f64(bits[1]), f64(bits[2])
    t0 = time.perf_counter()
    ro, rl = oatt.attention(q, k, v, "triangle", cfg["sink"], cfg["window"], cfg["last_q"])
    dt = time.perf_counter() - t0
    tri()
    torch.cuda.synchronize()
    err = error_vs_oracle((o.float().cpu().numpy(), lse.cpu().numpy()), (None, ro, rl))
    flops = 4.0 * 128 * 64 * cfg["d"] * plan.k_tile.size * cfg["Hq"] * cfg["B"]
    print(f"[bench] full-layer oracle: {dt:.1f} s on {threads} threads", file=sys.stderr, flush=True)
    return {"seconds": round(dt, 2), "cores": int(threads), "rows": int(q.shape[1] * q.shape[2]),
            "tflops": round(flops / dt / 1e12, 6), "gpu_layer_vs_oracle": err}


def error_vs_oracle(sample, ref):
    """Max and mean |dO|, max |dLSE| / max(1, |LSE|) of a sample against the
    oracle rows, and mean |O| of the oracle rows (the scale of the errors)."""
    o, l = sample
    _, ro, rl = ref
    err = np.abs(o - ro)
    return {"o_max_abs_err": float(f"{err.max():.3e}"), "o_mean_abs_err": float(f"{err.mean():.3e}"),
            "o_mean_abs_exact": float(f"{np.abs(ro).mean():.3e}"),
            "lse_max_rel_err": float(f"{(np.abs(l - rl) / np.maximum(1.0, np.abs(rl))).max():.3e}")}


def bench_dynamic(t, args, dense_ms, d, Hq, B, dev, stream):
    """The dense layer with dynamic block-sparse tile lists (probe queries
    against pooled keys, keep at alpha x max; FlashPrefill page 2.1-2.3):
    plan and list attention timed separately on the same inputs."""
    import static_triangle_sparse_amd as tsa
    plan = tsa.DynPlan(t, dev)
    plan_ms, _ = time_launches(lambda: plan.run(t, args.dyn_alpha, stream), args.dense_steps, 1)
    lists = lambda: tsa.tri_attn_prefill_lists(t, plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                                               plan.d_flags.data_ptr(), stream)
    attn_ms, _ = time_launches(lists, args.dense_steps, 1)
    nnz = int(plan.d_row_ptr[-1].item())
    kept_flops = 4.0 * 128 * 64 * d * nnz  # nnz already counts every (batch, head)
    total = plan_ms + attn_ms
    print(f"[bench] dynamic dense (alpha {args.dyn_alpha}): plan {plan_ms:.3f} ms + attention "
          f"{attn_ms:.3f} ms, density {nnz / plan.max_nnz:.4f}", file=sys.stderr, flush=True)
    return {"alpha": args.dyn_alpha, "plan_ms": round(plan_ms, 4), "attention_ms": round(attn_ms, 4),
            "total_ms": round(total, 4), "density": round(nnz / plan.max_nnz, 4),
            "kept_tflops": round(kept_flops / (attn_ms * 1e-3) / 1e12, 2),
            "speedup_vs_dense": round(dense_ms / total, 2),
            "inputs": "the same random N(0,1) tensors (near-uniform attention: density is high)"}


def bench_per_head(t, args, cfg, d, Hq, B, dev, stream):
    """The triangle layer with per-head boundaries (TriAttention page: each
    head's region as diagonal-distance boundaries): windows 512, 1024, 2048,
    4096 and sinks 0 / 128 cycling over the heads, last-Q as configured."""
    import torch
    import static_triangle_sparse_amd as tsa
    window = [512 << (h % 4) for h in range(Hq)]
    sink = [128 * (h % 2) for h in range(Hq)]
    plan = tsa.head_plan(cfg["N"], sink, window, cfg["last_q"], dev)
    run = lambda: tsa.tri_attn_prefill_heads(t, plan.mp, plan.d_sink.data_ptr(), plan.d_window.data_ptr(),
                                             plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                                             plan.d_flags.data_ptr(), stream)
    ms, _ = time_launches(run, args.steps, args.warmup)
    flops = 4.0 * 128 * 64 * d * plan.k_tile.size * B  # the plan lists every head
    tf = flops / (ms * 1e-3) / 1e12
    print(f"[bench] per-head triangle: {ms:.3f} ms/layer, {tf:.0f} TFLOP/s", file=sys.stderr, flush=True)
    out = {"windows": "512,1024,2048,4096 cycling", "sinks": "0,128 cycling", "ms": round(ms, 4),
           "kept_tiles": int(plan.k_tile.size), "tflops": round(tf, 2),
           "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
    # the same layer with every head's window 512: bound by the last-Q lists
    # unless they are split over workgroups (tri_attn_prefill_split)
    short = tsa.device_plan(cfg["N"], "triangle", cfg["sink"], 512, cfg["last_q"], dev)
    plain = lambda: tsa.tri_attn_prefill(t, short.mp, short.d_row_ptr.data_ptr(), short.d_k_tile.data_ptr(),
                                         short.d_flags.data_ptr(), stream)
    chunk = 128
    ws = tsa.split_workspace(tsa.tri_attn_split_workspace_size(t, short.mp, chunk), dev,
                             torch.cuda.current_stream(dev))
    split = lambda: tsa.tri_attn_prefill_split(t, short.mp, None, None, short.d_row_ptr.data_ptr(),
                                               short.d_k_tile.data_ptr(), short.d_flags.data_ptr(), chunk,
                                               ws.data_ptr(), ws.numel(), stream)
    plain_ms, _ = time_launches(plain, args.steps, args.warmup)
    split_ms, _ = time_launches(split, args.steps, args.warmup)
    print(f"[bench] window 512: {plain_ms:.3f} ms, last-Q lists split in chunks of {chunk}: {split_ms:.3f} ms",
          file=sys.stderr, flush=True)
    out["window512"] = {"ms": round(plain_ms, 4), "split_ms": round(split_ms, 4), "chunk_tiles": chunk,
                        "kept_tiles_per_head": int(short.k_tile.size),
                        "split_pct_bf16_peak": round(100 * 4.0 * 128 * 64 * d * short.k_tile.size * Hq * B /
                                                     (split_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    return out


def bench_tiered(t, args, cfg, plan, tri_ms, d, Hq, B, dev, stream, rows):
    """The triangle layer with precision tiers (TriAttention page: per-head
    diagonal-distance boundaries choose each tile's precision, 8-bit near and
    4-bit far): fp8 (e4m3) scores on key tiles at least --low-dist keys behind
    the query tile, fp4 (e2m1) from --fp4-dist, bf16 on the rest; then two more
    settings.  The fp8 and fp4 copies of K and the layers are timed
    separately.  Each setting's sample rows are kept for its error against
    the exact triangle layer (filled in once the oracle has run)."""
    import numpy as np
    import torch
    import static_triangle_sparse_amd as tsa
    qk = tsa.QuantizedK(t, dev, fp4=True)
    quant_ms, _ = time_launches(lambda: qk.run(t, stream), args.dense_steps, 1)
    rows_of = np.repeat(np.arange(plan.row_ptr.size - 1), np.diff(plan.row_ptr))
    dist_min = rows_of * 128 - (plan.k_tile.astype(np.int64) * 64 + 63)
    o = torch.empty((B, Hq, cfg["N"], d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, cfg["N"]), dtype=torch.float32, device=dev)
    tt = tsa.AttnTensors.from_buffer_copy(t)
    tt.o, tt.lse = o.data_ptr(), lse.data_ptr()
    tt.o_stride[:] = [o.stride(0), o.stride(1), o.stride(2)]
    tt.lse_stride[:] = [lse.stride(0), lse.stride(1)]
    tt.o_dtype = tsa.TRI_DTYPE_BF16
    samples = []

    def layer(low_dist, fp4_dist=None):
        d8 = torch.from_numpy(np.full(Hq, low_dist, np.int32)).to(dev)
        d4 = None if fp4_dist is None else torch.from_numpy(np.full(Hq, fp4_dist, np.int32)).to(dev)
        f4 = (None, None, None) if d4 is None else (d4.data_ptr(), qk.k4.data_ptr(), qk.scale4.data_ptr())
        run = lambda: tsa.tri_attn_prefill_tiered(tt, plan.mp, d8.data_ptr(), qk.k8.data_ptr(), qk.scale.data_ptr(),
                                                  *f4, plan.d_row_ptr.data_ptr(), plan.d_k_tile.data_ptr(),
                                                  plan.d_flags.data_ptr(), stream)
        ms, _ = time_launches(run, args.steps, args.warmup)
        torch.cuda.synchronize()
        n4 = int(np.sum(dist_min >= fp4_dist)) if fp4_dist is not None else 0
        n8 = int(np.sum(dist_min >= low_dist)) - (int(np.sum((dist_min >= low_dist) & (dist_min >= fp4_dist)))
                                                  if fp4_dist is not None else 0)
        out = {"fp8_from": low_dist, "fp4_from": fp4_dist, "ms": round(ms, 4),
               "fp8_tile_fraction": round(n8 / max(1, plan.k_tile.size), 4),
               "fp4_tile_fraction": round(n4 / max(1, plan.k_tile.size), 4),
               "speedup_vs_bf16_triangle": round(tri_ms / ms, 3)}
        if rows is not None:
            samples.append((out, sample_of(o, lse, rows)))
        return out
    flops = 4.0 * 128 * 64 * d * plan.k_tile.size * Hq * B
    main_ = layer(args.low_dist, args.fp4_dist if args.fp4_dist >= 0 else None)
    main_["kept_tflops_bf16_equivalent"] = round(flops / (main_["ms"] * 1e-3) / 1e12, 2)
    others = [layer(1024), layer(10 ** 6, 0)]
    print(f"[bench] tiered triangle (fp8 from {main_['fp8_from']}, fp4 from {main_['fp4_from']}): K to fp8 + fp4 "
          f"{quant_ms:.3f} ms, layer {main_['ms']:.3f} ms ({main_['speedup_vs_bf16_triangle']}x); "
          f"fp8 from 1024 only: {others[0]['ms']:.3f} ms; fp4 off the diagonal band: {others[1]['ms']:.3f} ms",
          file=sys.stderr, flush=True)
    return {"setting": main_, "other_settings": others, "quantize_fp8_fp4_ms": round(quant_ms, 4),
            "note": ("kept_tflops_bf16_equivalent counts fp8/fp4 tiles as bf16 work (4*128*64*d FLOPs); "
                     "errors are against the exact (fp64) triangle layer on the oracle sample rows")}, samples


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=sorted(CONFIGS))
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--per-head", type=int, default=1,
                    help="also time the triangle layer with per-head windows (0: skip)")
    ap.add_argument("--dyn-alpha", type=float, default=0.9,
                    help="keep threshold of the dynamic block-sparse dense layer (0 disables it)")
    ap.add_argument("--low-dist", type=int, default=0,
                    help="precision tiers: fp8 scores on key tiles at least this many keys behind "
                         "the query tile (negative: disable the tiered layers)")
    ap.add_argument("--fp4-dist", type=int, default=1024,
                    help="precision tiers: fp4 scores from this distance on (negative: no fp4 tier); "
                         "the default pair is the page's 8-bit-near, 4-bit-far scheme")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 2.5 s shader-clock run (profiling runs)")
    ap.add_argument("--full-oracle", action="store_true",
                    help="also time the fp64 oracle on every row of the layer (about a minute on 16 "
                         "host cores at 128K) and compare the whole layer with it")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer shards by KV-head group with no communication; see the design notes)",
              file=sys.stderr)
        return 2

    import torch
    import static_triangle_sparse_amd as tsa
    dev = torch.device("cuda:0")
    tsa.load()
    cfg = CONFIGS[args.config]
    print(f"[bench] config {args.config}: {cfg['name']}", file=sys.stderr, flush=True)

    if cfg["layers"]:
        return bench_stack(args, cfg, dev)

    (q, k, v), bits = make_layer_inputs(cfg, 0, dev)
    B, Hq, N, d = cfg["B"], cfg["Hq"], cfg["N"], cfg["d"]
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    # the host planner (sizing call + fill call), outside the timed region
    mp = tsa.mask_params(N, "triangle", cfg["sink"], cfg["window"], cfg["last_q"])
    tsa.tri_attn_plan(mp)
    t0 = time.perf_counter()
    plan_runs = 20
    for _ in range(plan_runs):
        tsa.tri_attn_plan(mp)
    plan_ms = (time.perf_counter() - t0) * 1e3 / plan_runs
    print(f"[bench] host planner: {plan_ms:.3f} ms", file=sys.stderr, flush=True)
    plan = tsa.device_plan(N, "triangle", cfg["sink"], cfg["window"], cfg["last_q"], dev)
    t = tsa.make_tensors(q, k, v, o, lse)
    stream = torch.cuda.current_stream(dev).cuda_stream
    tri = lambda: tsa.tri_attn_prefill(t, plan.mp, plan.d_row_ptr.data_ptr(),
                                       plan.d_k_tile.data_ptr(), plan.d_flags.data_ptr(), stream)
    dense = lambda: tsa.dense_causal_prefill(t, stream)

    tri_ms, tri_wall = time_launches(tri, args.steps, args.warmup)
    print(f"[bench] triangle: {tri_ms:.3f} ms/layer (wall {tri_wall:.3f})", file=sys.stderr, flush=True)
    tiles = kept_tiles_per_head(plan)
    flops = 4.0 * 128 * 64 * d * tiles * Hq * B
    tflops = flops / (tri_ms * 1e-3) / 1e12
    # per-launch spread, warm (back to back) and cold (caches flushed by a 512 MiB write)
    runs = {"warm": time_each(tri, max(20, args.steps)), "cold": time_each(tri, max(20, args.steps), 512)}
    runs["cold"]["flush"] = "512 MiB device write before each launch, outside the events"
    print(f"[bench] triangle per launch: warm median {runs['warm']['median_ms']:.3f} ms, cold median "
          f"{runs['cold']['median_ms']:.3f} ms", file=sys.stderr, flush=True)
    # the sample rows of the oracle baseline, kept for the error figures
    rows = None if args.no_cpu_baseline else sample_tiles(N)[1]
    torch.cuda.synchronize()
    tri_sample = sample_of(o, lse, rows) if rows is not None else None
    # the same launches for ~2.5 s more, with the shader clock read meanwhile:
    # the fraction of the MFMA peak at the clock the chip actually ran
    sclk, detail = (None, "skipped (--no-clock)") if args.no_clock else measure_clock(tri, tri_ms)
    at_clock = {"sclk_mhz": round(sclk, 1) if sclk else None, "how": detail}
    if sclk:
        peak_at = 256 * 4096 * sclk * 1e6 / 1e12
        at_clock.update(peak_tflops_at_sclk=round(peak_at, 1), pct_peak_at_sclk=round(100 * tflops / peak_at, 2))
    print(f"[bench] shader clock: {at_clock}", file=sys.stderr, flush=True)

    extra = {}
    if not args.no_dense:
        dense_ms, _ = time_launches(dense, args.dense_steps, 1)
        ctiles = causal_tiles_per_head(N)
        dflops = 4.0 * 128 * 64 * d * ctiles * Hq * B
        extra = {"dense_ms": round(dense_ms, 4),
                 "dense_tflops": round(dflops / (dense_ms * 1e-3) / 1e12, 2),
                 "dense_pct_peak": round(100 * dflops / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                 "triangle_speedup_vs_dense": round(dense_ms / tri_ms, 2),
                 "dense_kept_tiles_per_head": ctiles}
        print(f"[bench] dense causal: {dense_ms:.3f} ms/layer", file=sys.stderr, flush=True)
        if args.dyn_alpha > 0:
            extra["dynamic_dense"] = bench_dynamic(t, args, dense_ms, d, Hq, B, dev, stream)
    if args.per_head:
        extra["per_head_triangle"] = bench_per_head(t, args, cfg, d, Hq, B, dev, stream)
    tier_samples = []
    if args.low_dist >= 0:
        extra["tiered_triangle"], tier_samples = bench_tiered(t, args, cfg, plan, tri_ms, d, Hq, B, dev,
                                                              stream, rows)

    if args.calib_copy_mib:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.calib_copy_mib} MiB done", file=sys.stderr, flush=True)
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample) ...", file=sys.stderr, flush=True)
        cpu, ref = cpu_baseline(bits, cfg, plan)
        # the timed bf16 layer and each precision-tier setting against the exact
        # (fp64) triangle layer on the same rows
        extra["triangle_error_vs_oracle"] = error_vs_oracle(tri_sample, ref)
        for entry, sample in tier_samples:
            entry["error_vs_exact_triangle"] = error_vs_oracle(sample, ref)

    if args.full_oracle:
        extra["cpu_full_layer"] = full_oracle(bits, cfg, plan, tri, o, lse)

    traffic = read_traffic(args.config)
    out = {
        "metric": METRIC if args.config == 3 else
        f"triangle prefill ms + kept-tile TFLOP/s (% bf16 MFMA peak) at N={N}, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tri_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"] + " triangle prefill layer", "batch": B, "heads_q": Hq,
                   "heads_kv": cfg["Hkv"], "head_dim": d, "seqlen": N, "sink": cfg["sink"],
                   "window": cfg["window"], "last_q": cfg["last_q"], "tile": "128x64",
                   "o_dtype": "bf16", "kept_tiles_per_head": tiles},
        "triangle_ms": round(tri_ms, 4),
        "plan_ms": round(plan_ms, 4),
        "plan_note": "host planner, one tri_attn_plan sizing call plus one fill call, once per shape",
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "triangle_per_launch": runs,
        "measured_clock": at_clock,
        **extra,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_stack(args, cfg, dev):
    """Configs 4-5: every layer's attention back to back on one stream, layers
    before tri_start dense causal, the rest triangle."""
    import torch
    import static_triangle_sparse_amd as tsa
    B, Hq, Hkv, N, d, L = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["d"], cfg["layers"]
    layers = []
    for l in range(L):
        (q, k, v), _ = make_layer_inputs(cfg, 1000 + l, dev, host=False)
        layers.append((q, k, v))
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    descs = [tsa.make_tensors(q, k, v, o, lse) for (q, k, v) in layers]
    tsa.device_plan(N, "triangle", cfg["sink"], cfg["window"], cfg["last_q"], torch.cuda.current_device())
    modes = [tsa.layer_mode(l, cfg["tri_start"]) for l in range(L)]

    def step():
        tsa.stack_prefill(descs, cfg["tri_start"], cfg["sink"], cfg["window"], cfg["last_q"], stream)

    steps = max(1, min(args.steps, 3))
    ms, _ = time_launches(step, steps, min(args.warmup, 1))
    tiles = kept_tiles_per_head(tsa.device_plan(N, "triangle", cfg["sink"], cfg["window"], cfg["last_q"],
                                                torch.cuda.current_device()))
    ctiles = causal_tiles_per_head(N)
    n_dense = sum(m == "causal" for m in modes)
    flops = 4.0 * 128 * 64 * d * Hq * B * (n_dense * ctiles + (L - n_dense) * tiles)
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "TriangleMix layer-stack attention ms + kept-tile TFLOP/s, 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": min(args.warmup, 1), "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (torch device generator, seed 1000 + layer)",
        "config": {"workload": cfg["name"], "layers": L, "dense_layers": n_dense, "seqlen": N,
                   "heads_q": Hq, "heads_kv": Hkv, "head_dim": d},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
