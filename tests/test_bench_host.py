"""Host logic of bench.py (no GPU): the one-GPU guard, the workload configs,
the kept-tile counts the TFLOP/s figures divide by, the oracle sample, the
error summary, and the gating of the committed HBM-traffic figure on the
kernel source it was measured for."""
import numpy as np
import pytest

import bench
from oracle import mask as omask


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_configs_are_the_benchmark_workloads():
    # the five workloads: a tiny single head, the Llama-3-8B-shaped layer at 32K
    # and 128K, and the two layer stacks (shapes, mask parameters, layer split)
    c = bench.CONFIGS
    assert (c[1]["Hq"], c[1]["N"], c[1]["d"], c[1]["sink"], c[1]["window"], c[1]["last_q"]) == \
        (1, 512, 64, 64, 128, 64)
    for i, N in ((2, 32768), (3, 131072)):
        assert (c[i]["Hq"], c[i]["Hkv"], c[i]["N"], c[i]["d"]) == (32, 8, N, 128)
        assert (c[i]["sink"], c[i]["window"], c[i]["last_q"]) == (128, 2048, 128)
    assert (c[4]["layers"], c[4]["tri_start"], c[4]["N"]) == (32, 12, 65536)
    assert (c[5]["layers"], c[5]["tri_start"], c[5]["N"], c[5]["Hq"], c[5]["Hkv"]) == (28, 20, 131072, 28, 4)
    for i in (4, 5):
        assert (c[i]["d"], c[i]["sink"], c[i]["window"], c[i]["last_q"]) == (128, 128, 2048, 128)


@pytest.mark.parametrize("N", [1, 127, 128, 129, 1000, 32768])
def test_causal_tile_count_is_the_causal_plan(N):
    # the dense layer's kept tiles per head: every causal key tile of every query tile
    row_ptr = omask.interval_tiles(N, 128, 64, "causal")[0]
    assert bench.causal_tiles_per_head(N) == int(row_ptr[-1])


def test_causal_tile_counts_at_the_benchmark_sizes():
    assert bench.causal_tiles_per_head(131072) == 1049600
    assert bench.causal_tiles_per_head(32768) == 65792
    assert bench.causal_tiles_per_head(65536) == 262656


@pytest.mark.parametrize("N", [512, 32768, 131072])
def test_oracle_sample_tiles(N):
    tiles, rows = bench.sample_tiles(N)
    nq = -(-N // 128)
    fixed = {0, 1, 15, 16, 17, nq - 2, nq - 1} & set(range(nq))
    assert fixed <= set(tiles)
    assert tiles == sorted(set(tiles)) and all(0 <= t < nq for t in tiles)
    assert len(tiles) == min(nq, len(fixed) + 128)
    assert np.array_equal(rows, np.concatenate([np.arange(t * 128, min(N, t * 128 + 128)) for t in tiles]))
    assert bench.sample_tiles(N)[0] == tiles  # seeded


def test_error_summary():
    ro = np.array([[[[0.5, -1.0], [2.0, 0.0]]]])
    rl = np.array([[[0.5, -3.0]]])
    o = ro + np.array([[[[0.01, 0.0], [-0.03, 0.0]]]])
    lse = rl + np.array([[[0.002, 0.006]]])
    e = bench.error_vs_oracle((o, lse), (None, ro, rl))
    assert e["o_max_abs_err"] == pytest.approx(0.03)
    assert e["o_mean_abs_err"] == pytest.approx(0.01)
    assert e["o_mean_abs_exact"] == pytest.approx(0.875)
    # |dLSE| / max(1, |LSE|): 0.002 / 1 and 0.006 / 3
    assert e["lse_max_rel_err"] == pytest.approx(0.002)


def test_traffic_figure_follows_the_kernel_source(monkeypatch):
    kv = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    # the algorithmic bytes of the profile are Q and O (bf16, 32 heads), K and V
    # (bf16, 8 KV heads) and the f32 LSE of the 128K layer, each once
    N, d = 131072, 128
    assert float(kv["algorithmic_bytes_per_launch"]) == pytest.approx(
        2 * 32 * N * d * 2 + 2 * 8 * N * d * 2 + 4 * 32 * N, rel=1e-5)
    got = bench.read_traffic(bench.TRAFFIC_CONFIG)
    if kv["kernel_source_sha256_16"] == bench.kernel_hash():
        assert got == float(kv["hbm_bytes_per_launch"])
    else:
        assert got is None
    assert bench.read_traffic(2) is None  # taken on the 128K layer only
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.read_traffic(bench.TRAFFIC_CONFIG) is None
