"""The host-side parts of bench.py: the FLOP accounting it reports rates with,
the traffic stamp's staleness check, the single-GPU guard and the CPU baseline
leg on a tiny input (no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(T, S, W, is_local):
    off = S - T
    return sum(1 for t in range(T) for j in range(S)
               if j <= t + off and (not is_local or j > t + off - W))


@pytest.mark.parametrize("T,S,W,is_local", [
    (1, 1, 1, True), (10, 10, 3, True), (10, 10, 3, False), (7, 19, 5, True),
    (7, 19, 50, True), (33, 33, 33, True), (64, 100, 16, False)])
def test_prefill_pairs_counts_the_visible_pairs(T, S, W, is_local):
    assert bench.prefill_pairs(T, S, W, is_local) == brute_pairs(T, S, W, is_local)


@pytest.mark.parametrize("T,S,W,is_local", [
    (100, 100, 40, True), (100, 100, 40, False), (64, 200, 70, True), (33, 33, 1, True)])
def test_tile_pairs_cover_every_visible_pair_in_whole_tiles(T, S, W, is_local):
    """The tile model counts every key tile a wave's rows touch, whole: at least
    the visible pairs, at most one extra tile per row at each band edge."""
    vis = brute_pairs(T, S, W, is_local)
    tiles = bench.prefill_tile_pairs(T, S, W, is_local, rows_per_wave=32, bn=32)
    assert tiles % 32 == 0 and tiles >= vis
    assert tiles <= vis + T * 2 * 32 + 32 * 32


def test_9b_pair_flops_match_the_closed_form():
    """At T = S = 8192: global sees T(T+1)/2 pairs per slice, local
    W(W+1)/2 + (T-W)W with W = 4096."""
    T, W = 8192, 4096
    assert bench.prefill_pairs(T, T, W, False) == T * (T + 1) // 2
    assert bench.prefill_pairs(T, T, W, True) == W * (W + 1) // 2 + (T - W) * W


def test_traffic_stamp_is_ignored_once_the_sources_change(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    good = {"prefill_source_sha256": bench.kernel_source_hash("prefill"),
            "traffic_bytes_per_launch": 123}
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("prefill", "traffic_bytes_per_launch") == 123
    f.write_text(json.dumps(dict(good, prefill_source_sha256="0" * 64)))
    assert bench.measured_traffic("prefill", "traffic_bytes_per_launch") is None
    f.write_text("not json")
    assert bench.measured_traffic("prefill", "traffic_bytes_per_launch") is None


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def test_cpu_baseline_leg_on_a_tiny_input():
    from attention_g2attn_prefill_amd import synth
    cfg = dict(synth.WORKLOADS["tiny"])
    cfg["dtype"] = "bf16"
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, 64, 4, 64, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 64, 2, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 64, 2, 64, generator=g).to(torch.bfloat16)
    res = bench.cpu_baseline(dict(cfg, window=16), q, k, v, rows_per_layer=20)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1 and "20 seeded random" in res["sample"]
