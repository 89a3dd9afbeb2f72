"""Host-side accounting of bench.py (no GPU): the algorithmic FLOPs behind
the roofline line, the refusal of more than one GPU, and the gating of the
recorded HBM traffic on the library sources."""
import os
import subprocess
import sys

import numpy as np

import synth
from oracle import qv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _grids(wl):
    return [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]


def test_flops_448_closed_forms():
    wl = synth.W448
    total, per = bench.workload_flops(wl, _grids(wl), fold=True)
    n, d, f = 1024, 1280, 5120
    assert per["qkv"] == 2 * n * d * 3 * d == 10_066_329_600
    assert per["fc1"] == per["fc2"] == 2 * n * d * f == 13_421_772_800
    assert per["proj"] == 2 * n * d * d
    # softmax(q k^T) v per head: two n x n x 80 products, 16 heads
    assert per["attention"] == 16 * 2 * (2 * n * n * 80)
    assert per["patch_embed"] == 2 * n * (3 * 14 * 14) * d      # Conv2d fold: K = 588
    assert bench.workload_flops(wl, _grids(wl), fold=False)[1]["patch_embed"] == 2 * n * 1176 * d
    assert per["merge_fc1"] == 2 * 256 * 5120 * 5120 and per["merge_fc2"] == 2 * 256 * 5120 * 1536
    blocks = per["qkv"] + per["attention"] + per["proj"] + per["fc1"] + per["fc2"]
    assert total == per["patch_embed"] + 32 * blocks + per["merge_fc1"] + per["merge_fc2"]


def test_windowed_attention_flops_match_oracle_windows():
    """The windowed attention count equals sum over the oracle's own window
    groups of 4 d n_w^2 (an independent enumeration of the windows)."""
    wl = synth.WORKLOADS["qwen25vl_7b_3584_window"]
    grids = _grids(wl)
    _, per = bench.workload_flops(wl, grids)
    groups = O.window_groups(grids, wl.window)
    sizes = np.array([len(g) for g in groups])
    win = 4 * wl.dim * int((sizes.astype(np.int64) ** 2).sum())
    n = sum(t * h * w for t, h, w in grids)
    full = 4 * wl.dim * n * n
    nfull = len([b for b in wl.full_blocks if b < wl.depth])
    assert per["attention"] == (nfull * full + (wl.depth - nfull) * win) / wl.depth
    # 3584x3584: 256 x 256 patches in 8 x 8 windows -> 1024 windows of 64
    assert len(sizes) == 1024 and (sizes == 64).all()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_the_recorded_sources(monkeypatch):
    rec = bench.traffic_for("fc2", "qwen2vl_2b_448")
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.traffic_for("fc2", "qwen2vl_2b_448") is None
    if rec is not None:  # recorded for the sources in the tree: a plausible byte count
        assert 10e6 < rec < 1e9


def test_extrapolated_cpu_baseline_fields():
    """The sampled oracle baseline runs on the CPU and reports itself as
    extrapolated, with a positive rate and the sample it was scaled from."""
    wl = synth.small_workload("ex", [(224, 224, 1)], depth=2)
    params, imgs = synth.params(wl), synth.pixels(wl)
    r = bench.cpu_baseline_extrapolated(wl, params, imgs, rows=(32, 128), merge_groups=16)
    assert r["kind"] == "oracle" and r["extrapolated"] is True and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["seconds_estimated_forward"] > 0 and "extrapolated" in r["sample"]
