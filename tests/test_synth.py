"""The seeded input recipe: shapes, determinism, bf16-exact parameters."""
import numpy as np

import synth
from oracle import qv_oracle as O


def test_mixed_batch_draw():
    sides = synth.mixed_sides(0, 16)
    assert sides == [(1344, 308), (532, 672), (476, 896), (1232, 364), (700, 336), (280, 588),
                     (1316, 336), (1316, 644), (280, 756), (644, 504), (672, 756), (616, 1204),
                     (980, 952), (896, 980), (560, 308), (560, 1204)]
    grids = [O.grid_thw(h, w)[2] for h, w in sides]
    n = [t * gh * gw for t, gh, gw in grids]
    assert sum(n) == 39692 and sum(n) // 4 == 9923


def test_workload_token_counts():
    want = {"toy_112_fp32": (64, 16), "qwen2vl_2b_448": (1024, 256), "qwen2vl_2b_672x4_varlen": (9216, 2304),
            "mixed16_varlen_7b_merger": (39692, 9923), "maxres_3584": (65536, 16384),
            "qwen25vl_7b_3584_window": (65536, 16384), "video_448_16f": (8192, 2048)}
    for name, wl in synth.WORKLOADS.items():
        grids = [O.grid_thw(h, w, f)[2] for h, w, f in wl.images]
        n = sum(t * gh * gw for t, gh, gw in grids)
        assert (n, n // 4) == want[name]


def test_params_are_seeded_and_bf16_exact():
    wl = synth.small_workload("t", [(56, 56, 1)], depth=2)
    a = synth.params(wl)
    b = synth.params(wl)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k])
        assert np.array_equal(synth.round_bf16(a[k]), a[k])
    assert a["patch_w"].shape == (1280, 3, 2, 14, 14)
    assert a["blocks.1.qkv_w"].shape == (3840, 1280)
    assert a["merger.fc2_w"].shape == (1536, 5120)
    assert abs(a["blocks.0.ln1_w"].mean() - 1) < 0.01 and abs(a["blocks.0.fc1_w"].std() - 0.02) < 1e-3
    # a shallower draw keeps the merger's values
    c = synth.params(wl, depth=1)
    assert "blocks.1.qkv_w" not in c and np.array_equal(c["merger.fc1_w"], a["merger.fc1_w"])
    px = synth.pixels(wl)
    assert px[0].shape == (1, 3, 56, 56) and px[0].dtype == np.float32
    assert px[0].min() >= -1 and px[0].max() <= 1
